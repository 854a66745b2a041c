// pack.cpp -- host-side packers (canonical -> tiled device layout) and the
// affine INT4 quantizer.  Pure CPU code, caller-owned buffers.
#include <math.h>

#include <algorithm>
#include <cmath>
#include <string.h>

#include "layout.h"
#include "tt_internal.h"

namespace tt {
namespace {

// Write one MXFP4 tile.  crow/srow[r] point at canonical row r of the tile
// (NULL for a padding row); ps[r] is its postscale.
void pack_mx_tile(const MxGeom &g, const uint8_t *const crow[kTileRows],
                  const uint8_t *const srow[kTileRows],
                  const float ps[kTileRows], uint8_t *dst) {
    for (int64_t kk = 0; kk < g.units; ++kk) {
        int64_t qv = (kk == g.units - 1) ? g.qv_last : 4;
        for (int64_t q = 0; q < qv; ++q) {
            int64_t blk = 4 * kk + q;
            for (int r = 0; r < kTileRows; ++r) {
                uint8_t *o = dst + kUnitBytes * kk + 16 * (r + 16 * q);
                if (crow[r])
                    memcpy(o, crow[r] + 16 * blk, 16);
                else
                    memset(o, 0, 16);
            }
        }
    }
    uint8_t *sc = dst + g.scale_off;
    for (int64_t j = 0; j < g.groups; ++j) {
        for (int lane = 0; lane < 64; ++lane) {
            int r = lane % 16, q = lane / 16;
            for (int t = 0; t < 4; ++t) {
                int64_t kk = 4 * j + t, blk = 4 * kk + q;
                uint8_t e = kPadScale;
                if (kk < g.units && blk < g.nb && srow[r]) e = srow[r][blk];
                sc[kGroupBytes * j + 4 * lane + t] = e;
            }
        }
    }
    uint8_t *tr = dst + g.ps_off;
    memcpy(tr, ps, sizeof(float) * kTileRows);
    memset(tr + sizeof(float) * kTileRows, 0, kTrailerBytes - sizeof(float) * kTileRows);
}

tt_status check_mx_shape(int64_t n, int64_t k, const char *nname) {
    TT_TRY(check_range(n, 1, TT_MAX_ROWS, nname));
    TT_TRY(check_range(k, 32, TT_MAX_K, "k"));
    if (k % 32) return fail(TT_E_SHAPE, "k = %lld is not a multiple of 32", (long long)k);
    return TT_OK;
}

// Round an fp64 value to the nearest binary16 (ties to even) and return the
// bit pattern.  Works on the binary64 fields directly.
uint16_t f16_bits_from_f64(double v) {
    uint64_t b;
    memcpy(&b, &v, sizeof b);
    uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000);
    int bexp = static_cast<int>((b >> 52) & 0x7FF);
    uint64_t man = b & ((1ull << 52) - 1);
    if (bexp == 0x7FF) return sign | (man ? 0x7E00 : 0x7C00);
    if (bexp == 0) return sign;  // binary64 subnormals are far below 2^-25
    int e = bexp - 1023;
    if (e > 15) return sign | 0x7C00;
    uint64_t sig = man | (1ull << 52);
    int shift = (e >= -14) ? 42 : 42 + (-14 - e);
    if (shift >= 60) return sign;
    uint64_t kept = sig >> shift;
    uint64_t rem = sig & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (kept & 1))) ++kept;
    if (e < -14) return static_cast<uint16_t>(sign | kept);  // 1024 is 2^-14
    int E = e + 15;
    if (kept == 2048) {
        kept = 1024;
        ++E;
    }
    if (E >= 31) return sign | 0x7C00;
    return static_cast<uint16_t>(sign | (E << 10) | (kept - 1024));
}

double f16_bits_to_f64(uint16_t h) {
    int E = (h >> 10) & 31, F = h & 1023;
    double m = (E == 0) ? ldexp(static_cast<double>(F), -24)
                        : ldexp(static_cast<double>(1024 + F), E - 25);
    return (h & 0x8000) ? -m : m;
}

}  // namespace
}  // namespace tt

using namespace tt;

extern "C" {

int64_t tt_mxfp4_matrix_pack_bytes(int64_t n, int64_t k) {
    tt_status st = check_mx_shape(n, k, "n");
    if (st != TT_OK) return st;
    return ceil_div(n, kTileRows) * mx_geom(k).stride;
}

int64_t tt_mxfp4_gateup_pack_bytes(int64_t inter, int64_t hidden) {
    tt_status st = check_mx_shape(inter, hidden, "inter");
    if (st != TT_OK) return st;
    return ceil_div(inter, kTileRows / 2) * mx_geom(hidden).stride;
}

tt_status tt_pack_mxfp4_matrix(const uint8_t *codes, const uint8_t *scales,
                               const float *ps, int64_t n, int64_t k,
                               void *dst, int64_t dst_bytes) {
    TT_TRY(check_ptr(codes, "codes"));
    TT_TRY(check_ptr(scales, "scales"));
    TT_TRY(check_ptr(dst, "dst"));
    TT_TRY(check_mx_shape(n, k, "n"));
    const MxGeom g = mx_geom(k);
    const int64_t tiles = ceil_div(n, kTileRows);
    if (dst_bytes < tiles * g.stride)
        return fail(TT_E_SIZE, "dst holds %lld bytes, the pack needs %lld",
                    (long long)dst_bytes, (long long)(tiles * g.stride));
    uint8_t *out = static_cast<uint8_t *>(dst);
    for (int64_t t = 0; t < tiles; ++t) {
        const uint8_t *crow[kTileRows], *srow[kTileRows];
        float p[kTileRows];
        for (int r = 0; r < kTileRows; ++r) {
            int64_t row = t * kTileRows + r;
            bool ok = row < n;
            crow[r] = ok ? codes + row * (k / 2) : nullptr;
            srow[r] = ok ? scales + row * (k / 32) : nullptr;
            p[r] = ok ? (ps ? ps[row] : 1.0f) : 0.0f;
        }
        pack_mx_tile(g, crow, srow, p, out + t * g.stride);
    }
    clear_error();
    return TT_OK;
}

tt_status tt_pack_mxfp4_gateup(const uint8_t *g_codes, const uint8_t *g_scales,
                               const float *g_ps,
                               const uint8_t *u_codes, const uint8_t *u_scales,
                               const float *u_ps,
                               int64_t inter, int64_t hidden,
                               void *dst, int64_t dst_bytes) {
    TT_TRY(check_ptr(g_codes, "g_codes"));
    TT_TRY(check_ptr(g_scales, "g_scales"));
    TT_TRY(check_ptr(u_codes, "u_codes"));
    TT_TRY(check_ptr(u_scales, "u_scales"));
    TT_TRY(check_ptr(dst, "dst"));
    TT_TRY(check_mx_shape(inter, hidden, "inter"));
    const MxGeom g = mx_geom(hidden);
    const int64_t tiles = ceil_div(inter, kTileRows / 2);
    if (dst_bytes < tiles * g.stride)
        return fail(TT_E_SIZE, "dst holds %lld bytes, the pack needs %lld",
                    (long long)dst_bytes, (long long)(tiles * g.stride));
    uint8_t *out = static_cast<uint8_t *>(dst);
    for (int64_t t = 0; t < tiles; ++t) {
        const uint8_t *crow[kTileRows], *srow[kTileRows];
        float p[kTileRows];
        for (int i = 0; i < kTileRows / 2; ++i) {
            int64_t row = t * (kTileRows / 2) + i;
            bool ok = row < inter;
            crow[i] = ok ? g_codes + row * (hidden / 2) : nullptr;
            srow[i] = ok ? g_scales + row * (hidden / 32) : nullptr;
            p[i] = ok ? (g_ps ? g_ps[row] : 1.0f) : 0.0f;
            crow[i + 8] = ok ? u_codes + row * (hidden / 2) : nullptr;
            srow[i + 8] = ok ? u_scales + row * (hidden / 32) : nullptr;
            p[i + 8] = ok ? (u_ps ? u_ps[row] : 1.0f) : 0.0f;
        }
        pack_mx_tile(g, crow, srow, p, out + t * g.stride);
    }
    clear_error();
    return TT_OK;
}

// E2M1 rounding by midpoints: the index of the nearest of the magnitudes
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 is the number of midpoints below a, where a
// value sitting on a midpoint counts it only if the index above is even
// (ties to the even code); everything from 5 up (past the last midpoint)
// lands on 6.
static int fp4_index(double a) {
    static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    int idx = 0;
    for (int i = 0; i < 7; ++i) idx += (a > mid[i]) || (a == mid[i] && ((i + 1) & 1) == 0);
    return idx;
}

tt_status tt_quantize_mxfp4(const float *w, int64_t n, int64_t k, uint8_t *codes,
                            uint8_t *scales, float *ps) {
    TT_TRY(check_ptr(w, "w"));
    TT_TRY(check_ptr(codes, "codes"));
    TT_TRY(check_ptr(scales, "scales"));
    TT_TRY(check_range(n, 1, TT_MAX_ROWS, "n"));
    TT_TRY(check_range(k, 32, TT_MAX_K, "k"));
    if (k % 32) return fail(TT_E_SHAPE, "k = %lld is not a multiple of 32", (long long)k);
    for (int64_t i = 0; i < n * k; ++i)
        if (!std::isfinite(w[i]))
            return fail(TT_E_RANGE, "w[%lld][%lld] is not finite", (long long)(i / k),
                        (long long)(i % k));
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const int64_t nb = k / 32;
    for (int64_t r = 0; r < n; ++r) {
        const float *row = w + r * k;
        double num = 0.0, den = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const float *v = row + 32 * b;
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) amax = std::fmax(amax, std::fabs(v[j]));
            int e = amax == 0.0f ? -127 : std::ilogb(amax) - 2;
            e = std::min(127, std::max(-127, e));
            scales[r * nb + b] = static_cast<uint8_t>(e + 127);
            const double inv = std::ldexp(1.0, -e), sc = std::ldexp(1.0, e);
            uint8_t *crow = codes + r * (k / 2) + 16 * b;
            for (int j = 0; j < 32; j += 2) {
                uint8_t byte = 0;
                for (int h = 0; h < 2; ++h) {
                    const double x = static_cast<double>(v[j + h]) * inv;  // exact
                    const int idx = fp4_index(std::fabs(x));
                    const bool neg = std::signbit(x);
                    byte |= static_cast<uint8_t>((idx | (neg ? 8 : 0)) << (4 * h));
                    if (ps) {
                        const double d = (neg ? -mag[idx] : mag[idx]) * sc;
                        num += static_cast<double>(v[j + h]) * d;
                        den += d * d;
                    }
                }
                crow[j / 2] = byte;
            }
        }
        if (ps) ps[r] = den == 0.0 ? 1.0f : static_cast<float>(num / den);
    }
    clear_error();
    return TT_OK;
}

tt_status tt_quantize_int4_affine(const float *w, int64_t n, int64_t k,
                                  int64_t group, uint8_t *q, uint16_t *s,
                                  uint16_t *z) {
    TT_TRY(check_ptr(w, "w"));
    TT_TRY(check_ptr(q, "q"));
    TT_TRY(check_ptr(s, "s"));
    TT_TRY(check_ptr(z, "z"));
    TT_TRY(check_range(n, 1, TT_MAX_ROWS, "n"));
    TT_TRY(check_range(k, 2, TT_MAX_K, "k"));
    if (k % 2) return fail(TT_E_SHAPE, "k = %lld is odd", (long long)k);
    if (group != TT_INT4_GROUP)
        return fail(TT_E_SHAPE, "group = %lld; only %d is supported", (long long)group,
                    TT_INT4_GROUP);
    const int64_t G = ceil_div(k, group);
    // Check every scale first so that nothing is written on TT_E_RANGE.
    for (int64_t r = 0; r < n; ++r)
        for (int64_t gi = 0; gi < G; ++gi) {
            const float *row = w + r * k;
            int64_t a = gi * group, b = a + group < k ? a + group : k;
            double lo = 0.0, hi = 0.0;
            for (int64_t j = a; j < b; ++j) {
                double v = row[j];
                lo = v < lo ? v : lo;
                hi = v > hi ? v : hi;
            }
            uint16_t sb = f16_bits_from_f64((hi - lo) / 15.0);
            if ((sb & 0x7C00) == 0x7C00)
                return fail(TT_E_RANGE, "row %lld group %lld: scale %g overflows binary16",
                            (long long)r, (long long)gi, (hi - lo) / 15.0);
        }
    for (int64_t r = 0; r < n; ++r) {
        const float *row = w + r * k;
        uint8_t *qrow = q + r * (k / 2);
        memset(qrow, 0, static_cast<size_t>(k / 2));
        for (int64_t gi = 0; gi < G; ++gi) {
            int64_t a = gi * group, b = a + group < k ? a + group : k;
            double lo = 0.0, hi = 0.0;
            for (int64_t j = a; j < b; ++j) {
                double v = row[j];
                lo = v < lo ? v : lo;
                hi = v > hi ? v : hi;
            }
            uint16_t sb = f16_bits_from_f64((hi - lo) / 15.0);
            double sv = f16_bits_to_f64(sb);
            if (sv == 0.0) {
                sb = 0x3C00;
                sv = 1.0;
            }
            double zv = nearbyint(-lo / sv);
            zv = zv < 0.0 ? 0.0 : (zv > 15.0 ? 15.0 : zv);
            s[r * G + gi] = sb;
            z[r * G + gi] = f16_bits_from_f64(zv);
            for (int64_t j = a; j < b; ++j) {
                double qv = nearbyint(static_cast<double>(row[j]) / sv) + zv;
                qv = qv < 0.0 ? 0.0 : (qv > 15.0 ? 15.0 : qv);
                uint8_t c = static_cast<uint8_t>(qv);
                qrow[j >> 1] |= (j & 1) ? static_cast<uint8_t>(c << 4) : c;
            }
        }
    }
    clear_error();
    return TT_OK;
}

int64_t tt_fp8_pack_bytes(int64_t n, int64_t k) {
    tt_status st = check_range(n, 1, TT_MAX_ROWS, "n");
    if (st == TT_OK) st = check_range(k, 1, TT_MAX_K_FP8, "k");
    if (st != TT_OK) return st;
    return ceil_div(n, kF8TileRows) * f8_geom(k).stride;
}

tt_status tt_pack_fp8_matrix(const uint8_t *codes, const float *scale, int64_t n, int64_t k,
                             void *dst, int64_t dst_bytes) {
    TT_TRY(check_ptr(codes, "codes"));
    TT_TRY(check_ptr(dst, "dst"));
    int64_t need = tt_fp8_pack_bytes(n, k);
    if (need < 0) return static_cast<tt_status>(need);
    if (dst_bytes < need)
        return fail(TT_E_SIZE, "dst holds %lld bytes, the pack needs %lld",
                    (long long)dst_bytes, (long long)need);
    const F8Geom g = f8_geom(k);
    uint8_t *out = static_cast<uint8_t *>(dst);
    for (int64_t t = 0; t < ceil_div(n, kF8TileRows); ++t) {
        uint8_t *tb = out + t * g.stride;
        // unit u, lane l = r + 8 q: 16 codes of row r at k = 128 u + 16 q ..
        for (int64_t u = 0; u < g.units; ++u)
            for (int l = 0; l < 64; ++l) {
                const int64_t row = t * kF8TileRows + (l % 8);
                const int64_t k0 = kF8UnitK * u + 16 * (l / 8);
                uint8_t *o = tb + kUnitBytes * u + 16 * l;
                memset(o, 0, 16);
                if (row < n && k0 < k)
                    memcpy(o, codes + row * k + k0, static_cast<size_t>(std::min<int64_t>(16, k - k0)));
            }
        float sc[kF8TileRows];
        for (int r = 0; r < kF8TileRows; ++r) {
            const int64_t row = t * kF8TileRows + r;
            sc[r] = row < n ? (scale ? scale[row] : 1.0f) : 0.0f;
        }
        memset(tb + g.scale_off, 0, kF8TrailerBytes);
        memcpy(tb + g.scale_off, sc, sizeof(sc));
    }
    clear_error();
    return TT_OK;
}

int64_t tt_int4_pack_bytes(int64_t n, int64_t k, int64_t group) {
    tt_status st = check_range(n, 1, TT_MAX_ROWS, "n");
    if (st == TT_OK) st = check_range(k, 2, TT_MAX_K, "k");
    if (st != TT_OK) return st;
    if (k % 2) return fail(TT_E_SHAPE, "k = %lld is odd", (long long)k);
    if (group != TT_INT4_GROUP)
        return fail(TT_E_SHAPE, "group = %lld; only %d is supported", (long long)group,
                    TT_INT4_GROUP);
    return ceil_div(n, kTileRows) * i4_geom(k).stride;
}

// The scale stored for one group.  A group whose codes all equal its zero
// point holds only zero weights, s * (q - z) = +-0; storing a zero scale of
// the same sign keeps every decoded weight bit for bit and makes the matvec
// kernel's group term s * (sum (128 + q) x - (128 + z) sum x) exactly zero
// (the two sums are rounded in different orders and would otherwise leave a
// residue).  Non-finite scales are kept as they are.
static uint16_t int4_pack_scale(const uint8_t *q, int64_t row, int64_t rowbytes, int64_t k0,
                                int64_t k1, uint16_t s, uint16_t z) {
    if ((s & 0x7C00u) == 0x7C00u) return s;
    // z as a code: only a binary16 integer 0..15 can equal the codes
    int zc = -1;
    if ((z & 0x7FFFu) == 0) {
        zc = 0;
    } else if (!(z & 0x8000u)) {
        const int e = (z >> 10) & 31, m = z & 1023;
        if (e >= 15 && e <= 18 && (m & ((1 << (25 - e)) - 1)) == 0)
            zc = (1024 + m) >> (25 - e);
    }
    if (zc < 0) return s;
    for (int64_t kk = k0; kk < k1; ++kk) {
        const uint8_t b = q[row * rowbytes + (kk >> 1)];
        if (((kk & 1) ? (b >> 4) : (b & 15)) != zc) return s;
    }
    return static_cast<uint16_t>(s & 0x8000u);
}

tt_status tt_pack_int4(const uint8_t *q, const uint16_t *s, const uint16_t *z,
                       int64_t n, int64_t k, int64_t group, void *dst,
                       int64_t dst_bytes) {
    TT_TRY(check_ptr(q, "q"));
    TT_TRY(check_ptr(s, "s"));
    TT_TRY(check_ptr(z, "z"));
    TT_TRY(check_ptr(dst, "dst"));
    int64_t need = tt_int4_pack_bytes(n, k, group);
    if (need < 0) return static_cast<tt_status>(need);
    if (dst_bytes < need)
        return fail(TT_E_SIZE, "dst holds %lld bytes, the pack needs %lld",
                    (long long)dst_bytes, (long long)need);
    const I4Geom g = i4_geom(k);
    const int64_t G = ceil_div(k, group), rowbytes = k / 2;
    const int64_t tiles = ceil_div(n, kTileRows);
    uint8_t *out = static_cast<uint8_t *>(dst);
    for (int64_t t = 0; t < tiles; ++t) {
        uint8_t *tb = out + t * g.stride;
        for (int64_t kk = 0; kk < g.units; ++kk) {
            int64_t qv = (kk == g.units - 1) ? g.qv_last : 4;
            for (int64_t qq = 0; qq < qv; ++qq) {
                int64_t piece = 4 * kk + qq;
                for (int r = 0; r < kTileRows; ++r) {
                    int64_t row = t * kTileRows + r;
                    uint8_t *o = tb + kUnitBytes * kk + 16 * (r + 16 * qq);
                    memset(o, 0, 16);
                    if (row >= n) continue;
                    int64_t b0 = 16 * piece, b1 = b0 + 16 < rowbytes ? b0 + 16 : rowbytes;
                    if (b1 > b0) memcpy(o, q + row * rowbytes + b0, static_cast<size_t>(b1 - b0));
                }
            }
        }
        uint8_t *sz = tb + g.sz_off;
        for (int64_t j = 0; j < g.groups; ++j)
            for (int r = 0; r < kTileRows; ++r)
                for (int tt_ = 0; tt_ < 4; ++tt_) {
                    int64_t row = t * kTileRows + r, gi = 4 * j + tt_;
                    uint32_t v = 0;
                    if (row < n && gi < G) {
                        const int64_t k0 = gi * group, k1 = k0 + group < k ? k0 + group : k;
                        v = static_cast<uint32_t>(int4_pack_scale(q, row, rowbytes, k0, k1,
                                                                  s[row * G + gi],
                                                                  z[row * G + gi])) |
                            (static_cast<uint32_t>(z[row * G + gi]) << 16);
                    }
                    memcpy(sz + kGroupBytes * j + 16 * r + 4 * tt_, &v, 4);
                }
    }
    clear_error();
    return TT_OK;
}

}  // extern "C"
