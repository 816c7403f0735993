// Host-side packers: the NVFP4 encoder (fp32 -> canonical codes + E4M3
// scales) and the device record layouts of NVFP4, VQ, VQ8 and BF16 experts.
// Plain C++17, no device access.
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

namespace moeq {

namespace {

// Nearest E4M3 (OCP E4M3FN) byte for a finite v >= 0, ties to the even
// byte, saturating at 448.  Subnormals are m * 2^-9 (byte m); normals are
// (1 + m/8) * 2^(e-7) (byte e << 3 | m).
uint8_t e4m3_rne(double v) {
    if (v >= 448.0) return 0x7e;
    if (v < 0.015625) {                       // below the smallest normal 2^-6
        double m = std::nearbyint(v * 512.0);  // exact scaling, ties to even
        return (uint8_t)m;                     // m == 8 is the normal 2^-6 = byte 8
    }
    int e2;
    double fr = std::frexp(v, &e2);            // v = fr * 2^e2, fr in [0.5, 1)
    int e = e2 - 1;                            // v = (2 fr) * 2^e, 2 fr in [1, 2)
    double q = std::nearbyint((2.0 * fr - 1.0) * 8.0);
    int m = (int)q;
    if (m == 8) {
        m = 0;
        ++e;
    }
    int byte = ((e + 7) << 3) | m;
    return (uint8_t)(byte > 0x7e ? 0x7e : byte);
}

double e4m3_value(uint8_t b) {
    int e = (b >> 3) & 15, m = b & 7;
    double v = e == 0 ? std::ldexp((double)m, -9) : std::ldexp(1.0 + m / 8.0, e - 7);
    return (b & 0x80) ? -v : v;
}

// E2M1 magnitude index of a = |w| relative to scale S: nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6} * S, ties to the even index, saturating at 6.
// The comparisons use midpoint * S, which is exact in double.
inline int e2m1_index(double a, double S) {
    if (a <= 0.25 * S) return 0;
    if (a < 0.75 * S) return 1;
    if (a <= 1.25 * S) return 2;
    if (a < 1.75 * S) return 3;
    if (a <= 2.5 * S) return 4;
    if (a < 3.5 * S) return 5;
    if (a <= 5.0 * S) return 6;
    return 7;
}

}  // namespace

// NVFP4 record tile writer: rows [0, n) x inputs [0, kin) of canonical bytes
// into row groups rg_step*g + rg_off of a record with nkb tiles per group.
static void nv_tiles(const uint8_t* codes, const uint8_t* scales, int32_t n, int32_t kin,
                     int rg_step, int rg_off, uint8_t* rec) {
    const int64_t nkb = nv_tiles_k(kin);
    const int kc = kin / 2, ks = kin / 16;
    for (int g = 0; g < n / 16; ++g) {
        for (int64_t kb = 0; kb < nkb; ++kb) {
            uint8_t* tile = rec + ((int64_t)(g * rg_step + rg_off) * nkb + kb) * kNvTileBytes;
            std::memset(tile, 0, kNvTileBytes);
            for (int L = 0; L < 64; ++L) {
                const int row = 16 * g + (L & 15);
                const int k0 = (int)kb * kNvTileK + (L >> 4) * 32;
                for (int b = 0; b < 16; ++b) {
                    const int kbyte = k0 / 2 + b;
                    if (2 * kbyte < kin) tile[L * 16 + b] = codes[(int64_t)row * kc + kbyte];
                }
                for (int q = 0; q < 2; ++q) {
                    const int sb = k0 / 16 + q;
                    if (sb < ks) tile[kNvScaleOff + L * 2 + q] = scales[(int64_t)row * ks + sb];
                }
            }
        }
    }
}

static void vq_tiles(const uint16_t* codes, int32_t n, int32_t kin, int rg_step, int rg_off,
                     uint8_t* rec) {
    const int64_t nkb = vq_tiles_k(kin);
    const int ng = kin / 8;
    for (int g = 0; g < n / 16; ++g) {
        for (int64_t kb = 0; kb < nkb; ++kb) {
            uint8_t* tile = rec + ((int64_t)(g * rg_step + rg_off) * nkb + kb) * kVqTileBytes;
            std::memset(tile, 0, kVqTileBytes);
            for (int L = 0; L < 64; ++L) {
                const int row = 16 * g + (L & 15);
                const int g0 = ((int)kb * kVqTileK + (L >> 4) * 64) / 8;
                uint16_t* dst = reinterpret_cast<uint16_t*>(tile + L * 16);
                for (int s = 0; s < 8; ++s)
                    if (g0 + s < ng) dst[s] = codes[(int64_t)row * ng + g0 + s];
            }
        }
    }
}

static void vq8_tiles(const uint8_t* codes, int32_t n, int32_t kin, int32_t m, int rg_step,
                      int rg_off, uint8_t* rec) {
    const int64_t nkb = vq_tiles_k(kin);
    const int ng = kin / 8;
    const int64_t tb = (int64_t)kVq8TileBytesPerCode * m;
    for (int g = 0; g < n / 16; ++g) {
        for (int64_t kb = 0; kb < nkb; ++kb) {
            uint8_t* tile = rec + ((int64_t)(g * rg_step + rg_off) * nkb + kb) * tb;
            std::memset(tile, 0, (size_t)tb);
            for (int L = 0; L < 64; ++L) {
                const int row = 16 * g + (L & 15);
                const int g0 = ((int)kb * kVq8TileK + (L >> 4) * 64) / 8;
                uint8_t* dst = tile + (int64_t)L * 8 * m;
                for (int s = 0; s < 8; ++s)
                    if (g0 + s < ng)
                        for (int j = 0; j < m; ++j)
                            dst[m * s + j] = codes[((int64_t)row * ng + g0 + s) * m + j];
            }
        }
    }
}

// BF16 record tile writer (bf16 bits [n, kin], row-major).
static void bf16_tiles(const uint16_t* w, int32_t n, int32_t kin, int rg_step, int rg_off,
                       uint8_t* rec) {
    const int64_t nkb = bf16_tiles_k(kin);
    for (int g = 0; g < n / 16; ++g) {
        for (int64_t kb = 0; kb < nkb; ++kb) {
            uint8_t* tile = rec + ((int64_t)(g * rg_step + rg_off) * nkb + kb) * kBf16TileBytes;
            std::memset(tile, 0, kBf16TileBytes);
            for (int j = 0; j < 4; ++j)
                for (int L = 0; L < 64; ++L) {
                    const int row = 16 * g + (L & 15);
                    const int k0 = (int)kb * kBf16TileK + (L >> 4) * 32 + 8 * j;
                    uint16_t* dst = reinterpret_cast<uint16_t*>(tile + 1024 * j + 16 * L);
                    for (int i = 0; i < 8; ++i)
                        if (k0 + i < kin) dst[i] = w[(int64_t)row * kin + k0 + i];
                }
        }
    }
}

static int64_t bf16_rec_bytes(int which, int32_t H, int32_t I) {
    if (which == 0) return round_up(bf16_matrix_bytes(2 * I, H), 256);
    return round_up(bf16_matrix_bytes(H, I), 256);
}

// A bf16 weight the kernels can use as fp16: finite and |w| <= 65504 (the
// largest bf16 below 65520, where fp16 rounding would overflow, is 65280).
static bool bf16_fits_f16(uint16_t b) { return (b & 0x7fffu) < 0x4780u; }

static int64_t vq8_rec_bytes(int which, int32_t H, int32_t I, int32_t m) {
    if (which == 0) return round_up(vq8_codes_bytes(2 * I, H, m) + 2LL * I * 2, 256);
    return round_up(vq8_codes_bytes(H, I, m) + 2LL * H, 256);
}

static int64_t vq_rec_bytes(int which, int32_t H, int32_t I) {
    if (which == 0) return round_up(vq_codes_bytes(2 * I, H) + 2LL * I * 2, 256);
    return round_up(vq_codes_bytes(H, I) + 2LL * H, 256);
}

static int64_t nv_rec_bytes(int which, int32_t H, int32_t I) { return nv_record_bytes(which, H, I); }

}  // namespace moeq

using namespace moeq;

extern "C" {

int moe_quantize_nvfp4(const float* w, int32_t n, int32_t kin, uint8_t* codes,
                       uint8_t* scales) {
    if (!w || !codes || !scales) return fail(MOE_EINVAL, "moe_quantize_nvfp4: null pointer");
    if (n < 0 || kin <= 0 || kin % 16 != 0)
        return fail(MOE_EINVAL, "moe_quantize_nvfp4: need n >= 0, kin > 0, kin % 16 == 0");
    for (int64_t o = 0; o < n; ++o) {
        const float* row = w + o * kin;
        uint8_t* crow = codes + o * (kin / 2);
        uint8_t* srow = scales + o * (kin / 16);
        for (int b = 0; b < kin / 16; ++b) {
            const float* blk = row + 16 * b;
            double amax = 0.0;
            for (int i = 0; i < 16; ++i) {
                if (!std::isfinite(blk[i]))
                    return fail(MOE_EINVAL, "moe_quantize_nvfp4: non-finite weight");
                double a = std::fabs((double)blk[i]);
                if (a > amax) amax = a;
            }
            const uint8_t sb = e4m3_rne(amax / 6.0);
            srow[b] = sb;
            const double S = e4m3_value(sb);
            for (int i = 0; i < 16; i += 2) {
                int c[2];
                for (int q = 0; q < 2; ++q) {
                    const double v = (double)blk[i + q];
                    int m = S > 0.0 ? e2m1_index(std::fabs(v), S) : 0;
                    c[q] = m | ((v < 0.0 && m != 0) ? 8 : 0);
                }
                crow[8 * b + i / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
    return MOE_OK;
}

int moe_quantize_nvfp4_residual(const float* w, int32_t n, int32_t kin, int32_t shift,
                                uint8_t* bc, uint8_t* bs, uint8_t* rc, uint8_t* rs) {
    if (!w || !bc || !bs || !rc || !rs)
        return fail(MOE_EINVAL, "moe_quantize_nvfp4_residual: null pointer");
    if (shift < 0 || shift > 14)
        return fail(MOE_EINVAL, "moe_quantize_nvfp4_residual: shift must be in [0, 14]");
    int st = moe_quantize_nvfp4(w, n, kin, bc, bs);
    if (st) return st;
    // r = fp32((w - base) * 2^shift), the base value (an E2M1 value times its
    // E4M3 scale) and the product exact in double
    static const double kE2m1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    std::vector<float> r((size_t)n * kin);
    for (int64_t o = 0; o < n; ++o)
        for (int32_t k = 0; k < kin; ++k) {
            const uint8_t byte = bc[o * (kin / 2) + k / 2];
            const int c = (k & 1) ? byte >> 4 : byte & 15;
            const double S = e4m3_value(bs[o * (kin / 16) + k / 16]);
            const double q = ((c & 8) ? -1.0 : 1.0) * kE2m1[c & 7] * S;
            r[(size_t)o * kin + k] =
                (float)std::ldexp((double)w[(size_t)o * kin + k] - q, shift);
        }
    return moe_quantize_nvfp4(r.data(), n, kin, rc, rs);
}

size_t moe_record_bytes(int fmt, int which, int32_t H, int32_t I) {
    if (H <= 0 || I <= 0 || (which != 0 && which != 1)) return 0;
    if (fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_NVFP4R) {
        if (H % 16 || I % 16) return 0;
        return (size_t)nv_rec_bytes(which, H, I) * (fmt == MOE_FMT_NVFP4R ? 2 : 1);
    }
    if (fmt == MOE_FMT_VQ) {
        if (H % 16 || I % 16) return 0;   // row groups of 16 outputs; inputs in groups of 8
        return (size_t)vq_rec_bytes(which, H, I);
    }
    if (fmt == MOE_FMT_BF16) {
        if (H % 16 || I % 16) return 0;
        return (size_t)bf16_rec_bytes(which, H, I);
    }
    if (fmt >= MOE_FMT_VQ8_M1 && fmt <= MOE_FMT_VQ8_M3)
        return moe_record_bytes_vq8(which, H, I, fmt - MOE_FMT_VQ8_M1 + 1);
    return 0;
}

size_t moe_record_bytes_vq8(int which, int32_t H, int32_t I, int32_t m) {
    if (H <= 0 || I <= 0 || (which != 0 && which != 1) || m < 1 || m > MOE_VQ8_MAX_M) return 0;
    if (H % 16 || I % 16) return 0;
    return (size_t)vq8_rec_bytes(which, H, I, m);
}

// E4M3FN has no infinities; S.1111.111 is its only NaN (0x7F, 0xFF).
static bool e4m3_is_nan(uint8_t b) { return (b & 0x7F) == 0x7F; }
// fp16 exponent field all ones: an infinity or a NaN.
static bool f16_not_finite(uint16_t b) { return (b & 0x7C00) == 0x7C00; }

static bool any_e4m3_nan(const uint8_t* s, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (e4m3_is_nan(s[i])) return true;
    return false;
}
static bool any_f16_not_finite(const uint16_t* s, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (f16_not_finite(s[i])) return true;
    return false;
}

int moe_pack_nvfp4_expert(const uint8_t* gc, const uint8_t* gs, const uint8_t* uc,
                          const uint8_t* us, const uint8_t* dc, const uint8_t* ds, int32_t H,
                          int32_t I, uint8_t* w13, uint8_t* w2) {
    if (!gc || !gs || !uc || !us || !dc || !ds || !w13 || !w2)
        return fail(MOE_EINVAL, "moe_pack_nvfp4_expert: null pointer");
    if (H <= 0 || I <= 0 || H % 16 || I % 16)
        return fail(MOE_EUNSUPPORTED, "moe_pack_nvfp4_expert: H and I must be positive multiples of 16");
    const int64_t ns = (int64_t)I * (H / 16);   // scale bytes per gate/up/down matrix
    if (any_e4m3_nan(gs, ns) || any_e4m3_nan(us, ns) || any_e4m3_nan(ds, ns))
        return fail(MOE_EINVAL, "moe_pack_nvfp4_expert: a block scale is the E4M3 NaN byte");
    std::memset(w13, 0, (size_t)nv_rec_bytes(0, H, I));
    std::memset(w2, 0, (size_t)nv_rec_bytes(1, H, I));
    nv_tiles(gc, gs, I, H, 2, 0, w13);
    nv_tiles(uc, us, I, H, 2, 1, w13);
    nv_tiles(dc, ds, H, I, 1, 0, w2);
    return MOE_OK;
}

int moe_pack_nvfp4r_expert(const uint8_t* const base[6], const uint8_t* const res[6], int32_t H,
                           int32_t I, uint8_t* w13, uint8_t* w2) {
    if (!base || !res || !w13 || !w2) return fail(MOE_EINVAL, "moe_pack_nvfp4r_expert: null pointer");
    for (int i = 0; i < 6; ++i)
        if (!base[i] || !res[i]) return fail(MOE_EINVAL, "moe_pack_nvfp4r_expert: null pointer");
    int st = moe_pack_nvfp4_expert(base[0], base[1], base[2], base[3], base[4], base[5], H, I, w13,
                                   w2);
    if (st) return st;
    return moe_pack_nvfp4_expert(res[0], res[1], res[2], res[3], res[4], res[5], H, I,
                                 w13 + nv_rec_bytes(0, H, I), w2 + nv_rec_bytes(1, H, I));
}

int moe_pack_vq_expert(const uint16_t* gc, const uint16_t* gs, const uint16_t* uc,
                       const uint16_t* us, const uint16_t* dc, const uint16_t* ds, int32_t H,
                       int32_t I, uint8_t* w13, uint8_t* w2) {
    if (!gc || !gs || !uc || !us || !dc || !ds || !w13 || !w2)
        return fail(MOE_EINVAL, "moe_pack_vq_expert: null pointer");
    if (H <= 0 || I <= 0 || H % 16 || I % 16)
        return fail(MOE_EUNSUPPORTED, "moe_pack_vq_expert: H and I must be positive multiples of 16");
    if (any_f16_not_finite(gs, I) || any_f16_not_finite(us, I) || any_f16_not_finite(ds, H))
        return fail(MOE_EINVAL, "moe_pack_vq_expert: a per-row scale is not finite");
    std::memset(w13, 0, (size_t)vq_rec_bytes(0, H, I));
    std::memset(w2, 0, (size_t)vq_rec_bytes(1, H, I));
    vq_tiles(gc, I, H, 2, 0, w13);
    vq_tiles(uc, I, H, 2, 1, w13);
    vq_tiles(dc, H, I, 1, 0, w2);
    const int64_t c13 = vq_codes_bytes(2 * I, H);
    std::memcpy(w13 + c13, gs, (size_t)I * 2);
    std::memcpy(w13 + c13 + (size_t)I * 2, us, (size_t)I * 2);
    std::memcpy(w2 + vq_codes_bytes(H, I), ds, (size_t)H * 2);
    return MOE_OK;
}

int moe_pack_vq8_expert(const uint8_t* gc, const uint16_t* gs, const uint8_t* uc,
                        const uint16_t* us, const uint8_t* dc, const uint16_t* ds, int32_t H,
                        int32_t I, int32_t m, uint8_t* w13, uint8_t* w2) {
    if (!gc || !gs || !uc || !us || !dc || !ds || !w13 || !w2)
        return fail(MOE_EINVAL, "moe_pack_vq8_expert: null pointer");
    if (H <= 0 || I <= 0 || H % 16 || I % 16)
        return fail(MOE_EUNSUPPORTED, "moe_pack_vq8_expert: H and I must be positive multiples of 16");
    if (m < 1 || m > MOE_VQ8_MAX_M)
        return fail(MOE_EUNSUPPORTED, "moe_pack_vq8_expert: m must be 1, 2 or 3");
    if (any_f16_not_finite(gs, I) || any_f16_not_finite(us, I) || any_f16_not_finite(ds, H))
        return fail(MOE_EINVAL, "moe_pack_vq8_expert: a per-row scale is not finite");
    std::memset(w13, 0, (size_t)vq8_rec_bytes(0, H, I, m));
    std::memset(w2, 0, (size_t)vq8_rec_bytes(1, H, I, m));
    vq8_tiles(gc, I, H, m, 2, 0, w13);
    vq8_tiles(uc, I, H, m, 2, 1, w13);
    vq8_tiles(dc, H, I, m, 1, 0, w2);
    const int64_t c13 = vq8_codes_bytes(2 * I, H, m);
    std::memcpy(w13 + c13, gs, (size_t)I * 2);
    std::memcpy(w13 + c13 + (size_t)I * 2, us, (size_t)I * 2);
    std::memcpy(w2 + vq8_codes_bytes(H, I, m), ds, (size_t)H * 2);
    return MOE_OK;
}

int moe_pack_bf16_expert(const uint16_t* gate, const uint16_t* up, const uint16_t* down,
                         int32_t H, int32_t I, uint8_t* w13, uint8_t* w2) {
    if (!gate || !up || !down || !w13 || !w2)
        return fail(MOE_EINVAL, "moe_pack_bf16_expert: null pointer");
    if (H <= 0 || I <= 0 || H % 16 || I % 16)
        return fail(MOE_EUNSUPPORTED, "moe_pack_bf16_expert: H and I must be positive multiples of 16");
    const int64_t n = (int64_t)H * I;
    for (const uint16_t* m : {gate, up, down})
        for (int64_t i = 0; i < n; ++i)
            if (!bf16_fits_f16(m[i]))
                return fail(MOE_EINVAL,
                            "moe_pack_bf16_expert: a weight is not finite or exceeds 65504");
    std::memset(w13, 0, (size_t)bf16_rec_bytes(0, H, I));
    std::memset(w2, 0, (size_t)bf16_rec_bytes(1, H, I));
    bf16_tiles(gate, I, H, 2, 0, w13);
    bf16_tiles(up, I, H, 2, 1, w13);
    bf16_tiles(down, H, I, 1, 0, w2);
    return MOE_OK;
}

static bool known_fmt(int f) { return f >= MOE_FMT_NVFP4 && f <= MOE_FMT_MAX; }

size_t moe_rot_sign_bytes(int32_t H, int32_t I) {
    if (H <= 0 || I <= 0 || H % 8 || I % 8) return 0;
    return (size_t)(2 * (int64_t)H + 3 * (int64_t)I) / 8;
}

int moe_pack_rot_signs(const int8_t* s_in13, const int8_t* s_og, const int8_t* s_ou,
                       const int8_t* s_in2, const int8_t* s_o2, int32_t H, int32_t I,
                       uint8_t* out) {
    if (!s_in13 || !s_og || !s_ou || !s_in2 || !s_o2 || !out)
        return fail(MOE_EINVAL, "moe_pack_rot_signs: null pointer");
    if (!moe_rot_sign_bytes(H, I)) return fail(MOE_EINVAL, "moe_pack_rot_signs: bad H or I");
    const int8_t* sec[5] = {s_in13, s_og, s_ou, s_in2, s_o2};
    const int32_t len[5] = {H, I, I, I, H};
    uint8_t* o = out;
    for (int q = 0; q < 5; ++q) {
        for (int32_t b = 0; b < len[q] / 8; ++b) {
            uint8_t byte = 0;
            for (int i = 0; i < 8; ++i) {
                const int8_t v = sec[q][8 * b + i];
                if (v != 1 && v != -1)
                    return fail(MOE_EINVAL, "moe_pack_rot_signs: a sign is not +1 or -1");
                if (v < 0) byte |= (uint8_t)(1u << i);
            }
            *o++ = byte;
        }
    }
    return MOE_OK;
}

// v <- R v for one vector: signs, then per block of b entries the Hadamard
// butterflies and 1/sqrt(b) (fp64).
static void rotate_vec(double* v, int32_t n, const int8_t* s, int32_t b) {
    const double norm = 1.0 / std::sqrt((double)b);
    for (int32_t i = 0; i < n; ++i) v[i] *= s[i];
    for (int32_t b0 = 0; b0 < n; b0 += b) {
        double* w = v + b0;
        for (int len = 1; len < b; len <<= 1)
            for (int i = 0; i < b; i += 2 * len)
                for (int j = i; j < i + len; ++j) {
                    const double a = w[j], c = w[j + len];
                    w[j] = a + c;
                    w[j + len] = a - c;
                }
        for (int i = 0; i < b; ++i) w[i] *= norm;
    }
}

static bool rot_block_ok(int32_t b) { return b == MOE_ROT_BLOCK || b == MOE_ROT_BLOCK_WIDE; }

int moe_rotate_matrix_blocks(const float* w, int32_t n_out, int32_t n_in, const int8_t* s_out,
                             const int8_t* s_in, int32_t block_out, int32_t block_in,
                             float* out) {
    if (!w || !s_out || !s_in || !out) return fail(MOE_EINVAL, "moe_rotate_matrix: null pointer");
    if (!rot_block_ok(block_out) || !rot_block_ok(block_in))
        return fail(MOE_EINVAL, "moe_rotate_matrix: a block must be 128 or 512");
    if (n_out <= 0 || n_in <= 0 || n_out % block_out || n_in % block_in)
        return fail(MOE_EINVAL, "moe_rotate_matrix: sizes must be positive multiples of the blocks");
    for (int32_t i = 0; i < n_in; ++i)
        if (s_in[i] != 1 && s_in[i] != -1) return fail(MOE_EINVAL, "moe_rotate_matrix: bad sign");
    for (int32_t i = 0; i < n_out; ++i)
        if (s_out[i] != 1 && s_out[i] != -1) return fail(MOE_EINVAL, "moe_rotate_matrix: bad sign");
    std::vector<double> m((size_t)n_out * n_in);
    for (size_t i = 0; i < m.size(); ++i) m[i] = w[i];
    for (int32_t o = 0; o < n_out; ++o)                                               // W R_in^T
        rotate_vec(&m[(size_t)o * n_in], n_in, s_in, block_in);
    std::vector<double> col(n_out);
    for (int32_t c = 0; c < n_in; ++c) {                                               // R_out (.)
        for (int32_t o = 0; o < n_out; ++o) col[o] = m[(size_t)o * n_in + c];
        rotate_vec(col.data(), n_out, s_out, block_out);
        for (int32_t o = 0; o < n_out; ++o) m[(size_t)o * n_in + c] = col[o];
    }
    for (size_t i = 0; i < m.size(); ++i) out[i] = (float)m[i];
    return MOE_OK;
}

int moe_rotate_matrix(const float* w, int32_t n_out, int32_t n_in, const int8_t* s_out,
                      const int8_t* s_in, float* out) {
    return moe_rotate_matrix_blocks(w, n_out, n_in, s_out, s_in, MOE_ROT_BLOCK, MOE_ROT_BLOCK,
                                    out);
}

int moe_record_table(const uint8_t* fmt_host, int32_t E, int32_t* rec, int32_t* n_by_fmt) {
    if (!fmt_host || !rec) return fail(MOE_EINVAL, "moe_record_table: null pointer");
    if (E < 1 || E > MOE_MAX_E) return fail(MOE_EINVAL, "moe_record_table: bad E");
    int32_t cnt[kNumFmt] = {};
    for (int e = 0; e < E; ++e) {
        const int f = fmt_host[e];
        if (!known_fmt(f))
            return fail(MOE_EUNSUPPORTED,
                        "moe_record_table: expert " + std::to_string(e) + " has unknown format tag " +
                            std::to_string(f));
        rec[e] = (f << 24) | cnt[f]++;
    }
    if (n_by_fmt)
        for (int f = 0; f < kNumFmt; ++f) n_by_fmt[f] = cnt[f];
    return MOE_OK;
}

int moe_record_table_resident(const uint8_t* fmt_host, int32_t E, int32_t* rec) {
    if (!fmt_host || !rec) return fail(MOE_EINVAL, "moe_record_table_resident: null pointer");
    if (E < 1 || E > MOE_MAX_E) return fail(MOE_EINVAL, "moe_record_table_resident: bad E");
    for (int e = 0; e < E; ++e) {
        const int f = fmt_host[e];
        if (!known_fmt(f))
            return fail(MOE_EUNSUPPORTED, "moe_record_table_resident: expert " + std::to_string(e) +
                                              " has unknown format tag " + std::to_string(f));
        rec[e] = (f << 24) | e;
    }
    return MOE_OK;
}

}  // extern "C"
