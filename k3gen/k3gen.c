/* k3gen: seeded, counter-based synthetic inputs. See k3gen.h for the contract. */
#include "k3gen.h"

#include <math.h>
#include <string.h>

#define K3G_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t k3g_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t k3g_hash(uint64_t seed, uint32_t tensor, uint64_t idx)
{
    /* stream start: one splitmix64 step of (seed, tensor); then step idx + 1 of that stream */
    const uint64_t s = k3g_mix(seed + K3G_GOLDEN * ((uint64_t)tensor + 1u));
    return k3g_mix(s + K3G_GOLDEN * (idx + 1u));
}

static inline double k3g_unit_open0(uint64_t h) /* (0, 1] */
{
    return ((double)(h >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}

static inline double k3g_unit(uint64_t h) /* [0, 1) */
{
    return (double)(h >> 11) * (1.0 / 9007199254740992.0);
}

static inline double k3g_normal_at(uint64_t seed, uint32_t tensor, uint64_t i)
{
    /* Box-Muller, cosine branch only; two draws per element */
    const double u1 = k3g_unit_open0(k3g_hash(seed, tensor, 2u * i));
    const double u2 = k3g_unit(k3g_hash(seed, tensor, 2u * i + 1u));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static inline uint16_t k3g_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) /* inf / nan: keep, quiet nan */
        return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x0040u : 0u));
    const uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

void k3g_normal_f32(float *out, size_t n, uint64_t seed, uint32_t tensor,
                    uint64_t idx0, double std)
{
#pragma omp parallel for schedule(static) if (n > 65536)
    for (size_t i = 0; i < n; i++)
        out[i] = (float)(std * k3g_normal_at(seed, tensor, idx0 + i));
}

void k3g_normal_bf16(uint16_t *out, size_t n, uint64_t seed, uint32_t tensor,
                     uint64_t idx0, double std)
{
#pragma omp parallel for schedule(static) if (n > 65536)
    for (size_t i = 0; i < n; i++)
        out[i] = k3g_f32_to_bf16((float)(std * k3g_normal_at(seed, tensor, idx0 + i)));
}

void k3g_uniform_f32(float *out, size_t n, uint64_t seed, uint32_t tensor,
                     uint64_t idx0, double lo, double hi)
{
#pragma omp parallel for schedule(static) if (n > 65536)
    for (size_t i = 0; i < n; i++)
        out[i] = (float)(lo + (hi - lo) * k3g_unit(k3g_hash(seed, tensor, idx0 + i)));
}

void k3g_bytes(uint8_t *out, size_t n, uint64_t seed, uint32_t tensor, uint64_t idx0)
{
    /* byte f of the tensor is byte (f % 8) of the draw at counter f / 8; whole 8-byte
     * words are produced from one draw */
    size_t head = (size_t)((8u - (idx0 & 7u)) & 7u);
    if (head > n) head = n;
    for (size_t i = 0; i < head; i++) {
        const uint64_t f = idx0 + i;
        out[i] = (uint8_t)(k3g_hash(seed, tensor, f >> 3) >> (8u * (unsigned)(f & 7u)));
    }
    const size_t words = (n - head) / 8;
    const uint64_t w0 = (idx0 + head) >> 3;
#pragma omp parallel for schedule(static) if (words > 8192)
    for (size_t k = 0; k < words; k++) {
        const uint64_t h = k3g_hash(seed, tensor, w0 + k);
        uint8_t *o = out + head + 8 * k;
        for (unsigned b = 0; b < 8; b++) o[b] = (uint8_t)(h >> (8u * b));
    }
    for (size_t i = head + 8 * words; i < n; i++) {
        const uint64_t f = idx0 + i;
        out[i] = (uint8_t)(k3g_hash(seed, tensor, f >> 3) >> (8u * (unsigned)(f & 7u)));
    }
}

void k3g_int_range_u8(uint8_t *out, size_t n, uint64_t seed, uint32_t tensor,
                      uint64_t idx0, int lo, int hi)
{
    const uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for schedule(static) if (n > 65536)
    for (size_t i = 0; i < n; i++)
        out[i] = (uint8_t)(lo + (int)((k3g_hash(seed, tensor, idx0 + i) >> 32) % span));
}
