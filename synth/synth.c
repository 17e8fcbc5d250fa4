/*
 * synth.c -- seeded, counter-based synthetic input tensors.
 *
 * Shared by the tests, the benchmark and the oracle's callers so that the CPU
 * oracle and the HIP library see identical input bytes.  Holds none of the
 * quantization arithmetic: only random numbers and rounding to the storage
 * dtype.
 *
 * Element i of a tensor (seed, stream) is a pure function of (seed, stream,
 * i), so any slice can be regenerated alone and the result does not depend on
 * the thread count.
 *   uniform:  u(j) = (splitmix64(key(seed, stream, j)) >> 11 + 0.5) * 2^-53,
 *             splitmix64 being Steele, Lea & Flood's 64-bit finaliser.
 *   normal:   Box-Muller on the pair (u(2p), u(2p+1)), p = i / 2; element
 *             2p takes r cos(t), element 2p+1 takes r sin(t).
 *   outlier:  an independent uniform on stream ^ OUTLIER_TAG; if it is below
 *             p_out the value is multiplied by out_mult.
 * The value is formed in double, rounded to fp32 (nearest even), and for
 * bf16 rounded again from fp32 to bf16 (nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OUTLIER_TAG 0x6F75746C69657273ull /* "outliers" */

static inline uint64_t splitmix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t key(uint64_t seed, uint64_t stream, uint64_t j)
{
    return splitmix64(seed * 0xD1B54A32D192ED03ull ^ splitmix64(stream)) + j * 0x9E3779B97F4A7C15ull;
}

static inline double u01(uint64_t seed, uint64_t stream, uint64_t j)
{
    return ((double)(splitmix64(key(seed, stream, j)) >> 11) + 0.5) * 0x1.0p-53;
}

static inline double normal_at(uint64_t seed, uint64_t stream, uint64_t i)
{
    uint64_t p = i >> 1;
    double u1 = u01(seed, stream, 2 * p), u2 = u01(seed, stream, 2 * p + 1);
    double r = sqrt(-2.0 * log(u1)), t = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(t) : r * cos(t);
}

static inline double value_at(uint64_t seed, uint64_t stream, uint64_t i, double sigma,
                              double p_out, double out_mult)
{
    double v = sigma * normal_at(seed, stream, i);
    if (p_out > 0.0 && u01(seed, stream ^ OUTLIER_TAG, i) < p_out) v *= out_mult;
    return v;
}

static inline uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Elements [start, start + count) of a N(0, sigma^2) tensor with outliers,
 * as fp32. */
void synth_normal_f32(float* out, int64_t start, int64_t count, uint64_t seed, uint64_t stream,
                      double sigma, double p_out, double out_mult)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i)
        out[i] = (float)value_at(seed, stream, (uint64_t)(start + i), sigma, p_out, out_mult);
}

/* Same, stored as bf16 bits. */
void synth_normal_bf16(uint16_t* out, int64_t start, int64_t count, uint64_t seed,
                       uint64_t stream, double sigma, double p_out, double out_mult)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i)
        out[i] = f32_to_bf16_bits((float)value_at(seed, stream, (uint64_t)(start + i), sigma,
                                                  p_out, out_mult));
}

/* Rows [row0, row0 + nrows) of a rows x k bf16 matrix whose rows fall into
 * `bands` equal contiguous bands; band b uses sigma_alt when b % period ==
 * phase, else sigma.  Element (r, c) is element r*k + c of the stream. */
void synth_banded_bf16(uint16_t* out, int64_t row0, int64_t nrows, int64_t rows, int64_t k,
                       uint64_t seed, uint64_t stream, int64_t bands, int64_t period,
                       int64_t phase, double sigma, double sigma_alt, double p_out,
                       double out_mult)
{
    int64_t i, n = nrows * k, band_rows = rows / bands;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        int64_t r = row0 + i / k, band = r / band_rows;
        double sg = (band % period == phase) ? sigma_alt : sigma;
        out[i] = f32_to_bf16_bits(
            (float)value_at(seed, stream, (uint64_t)(row0 * k + i), sg, p_out, out_mult));
    }
}
