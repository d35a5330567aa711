/* Seeded synthetic inputs, host side, in C for speed.
 *
 * Same definition as synth/gen.py: value i of stream s under seed k comes from
 * one Philox4x32-10 call (Salmon et al., SC'11, section 3) with counter
 * (i_lo, i_hi, s_lo, s_hi) and key (k_lo, k_hi); the eight 16-bit halves of its
 * output are summed (exact integer Irwin-Hall sum), centred by 262140,
 * converted to float exactly and multiplied once by the fp32 constant c.
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math, no FMA contraction). */
#include <stdint.h>
#include <stddef.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void philox10(uint32_t c[4], uint32_t k0, uint32_t k1)
{
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
        uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
}

void synth_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    philox10(c, key[0], key[1]);
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

static inline int32_t ih_centred(uint64_t seed, uint64_t stream, uint64_t i)
{
    uint32_t c[4] = {(uint32_t)i, (uint32_t)(i >> 32), (uint32_t)stream, (uint32_t)(stream >> 32)};
    philox10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    int32_t s = 0;
    for (int w = 0; w < 4; ++w) s += (int32_t)(c[w] & 0xFFFFu) + (int32_t)(c[w] >> 16);
    return s - 262140;
}

/* out[j] = float(S(start + j) - 262140) * scale, j < n (fp32 multiply). */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, int64_t n,
                      float scale, float *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        float z = (float)ih_centred(seed, stream, start + (uint64_t)j);
        out[j] = z * scale;
    }
}
