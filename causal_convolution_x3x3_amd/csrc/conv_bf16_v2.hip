// bf16 3x3x3 causal conv on gfx950 MFMA, register-blocked ("v2" family).
//
// Same GEMM view as conv_bf16.hip (M = output pixels, N = output channels,
// K = Cin x taps), built for throughput on the 3x3 spatial kernels that carry
// almost all of the decoder's FLOPs:
//
// * One workgroup of 8 waves per CU, two per SIMD so that one wave's LDS and
//   barrier waits are covered by the other's MFMAs.  Four waves along M each own
//   8 output rows x 16 columns (up_s = 1) or 2 source rows x 16 source columns at
//   all four output phases (up_s = 2) -- 128 output pixels; the two waves along
//   N split the NTILE output channels.
// * K is walked in steps of (temporal tap a, 32 channels); each step in three
//   sub-steps, one per spatial column tap d.  A sub-step needs the step's input
//   tile (A, in LDS for the whole step) and the weights of the three taps (b, d),
//   b = 0..2 (B, 3 x NTILE x 32).  Both are double-buffered in LDS; the next
//   sub-step's B and the next step's A are fetched into registers while the
//   current sub-step runs, then written to the idle buffers: one barrier per
//   sub-step.
// * A fragments are reused from registers.  up_s = 1: the fragment of LDS row s
//   (shifted by d) serves output rows s-b for the three row taps b.  up_s = 2:
//   with nearest upsampling, output phase (p, q) and tap (b, d) read source
//   offset (floor((p+b-1)/2), floor((q+d-1)/2)); a sub-step loads the fragments
//   of its (at most two) column offsets for the three row offsets and applies
//   each to every (phase, tap) pair that maps to it.  Every MFMA of the 27-tap
//   definition is still executed (the FLOP count is the algorithmic one); only
//   LDS reads are shared.
// * Work items (tile, frame, channel block) are dealt to the 8 XCDs in contiguous
//   ranges, so neighbouring tiles and consecutive frames (which share input rows
//   and frames) run under the same L2.
#include "cc3d_kernels.h"

namespace cc3d {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ const uint16_t* zframe(const ZWindow& z, int zi) {
    const int hist = z.kt - 1;
    if (zi < hist) {
        if (!z.first) return (const uint16_t*)z.cache + (int64_t)zi * z.frame_elems;
        return z.zero_hist ? nullptr : (const uint16_t*)z.x;
    }
    const int u = zi - hist;
    const int src = (z.up_t == 2) ? ((u + z.first) >> 1) : u;
    return (const uint16_t*)z.x + (int64_t)src * z.frame_elems;
}

// Work item of this workgroup: contiguous ranges of (tile, frame, channel block)
// per XCD (workgroups are dealt to the XCDs round-robin).
__device__ __forceinline__ bool decode_work(int ntiles, int t_out, int nblocks, int& tile, int& t, int& nb) {
    const int total = ntiles * t_out * nblocks;
    const int per_xcd = (total + 7) >> 3;
    const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (w >= total) return false;
    nb = w % nblocks;
    const int rest = w / nblocks;
    t = rest % t_out;
    tile = rest / t_out;
    return true;
}

// Geometry of the two variants (per group of four waves along M).
template <int UP>
struct Geo;
template <>
struct Geo<1> {  // tile: 8 output rows x 64 columns; M-wave w: columns 16w..16w+15
    static constexpr int TS_H = 8, TS_W = 64;
    static constexpr int MF = 8;  // M fragments per wave: one per row
};
template <>
struct Geo<2> {  // tile: 8 source rows x 16 source columns; M-wave w: source rows 2w, 2w+1
    static constexpr int TS_H = 8, TS_W = 16;
    static constexpr int MF = 8;  // 2 rows x 4 phases
};

// WN = waves along N: the workgroup has 4*WN waves (two per SIMD when WN = 2);
// wave (wm, wn) computes M-wave wm's pixels for the NF/WN fragments of half wn.
template <int UP, int NF, int WN>
__global__ __launch_bounds__(256 * WN, 1) void conv3_v2_kernel(ConvArgs a)
{
    using G = Geo<UP>;
    constexpr int NT = 256 * WN;        // threads
    constexpr int NFW = NF / WN;        // N fragments per wave
    constexpr int LH = G::TS_H + 2, LW = G::TS_W + 2;
    constexpr int NTILE = 16 * NF;
    constexpr int A_CH = LH * LW * 4;   // 16-byte chunks of one input tile (32 channels)
    constexpr int B_CH = 3 * NTILE * 4; // 16-byte chunks of one column tap's weights
    constexpr int A_IT = (A_CH + NT - 1) / NT;
    constexpr int B_IT = (B_CH + NT - 1) / NT;
    constexpr int MF = G::MF;
    static_assert(NF % WN == 0, "N fragments split evenly over the N waves");

    __shared__ uint4 lds_a[2][A_CH];
    __shared__ uint4 lds_b[2][B_CH];

    const int tiles_w = (a.w_in + G::TS_W - 1) / G::TS_W;
    const int tiles_h = (a.h_in + G::TS_H - 1) / G::TS_H;
    int tile, t, nb;
    if (!decode_work(tiles_w * tiles_h, a.t_out, a.nblocks, tile, t, nb)) return;
    const int i0 = (tile / tiles_w) * G::TS_H;  // source tile origin
    const int j0 = (tile % tiles_w) * G::TS_W;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;
    const int g = lane >> 4, k16 = lane & 15;

    f32x4 acc[MF][NFW];
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
        for (int f = 0; f < NFW; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = a.kt * a.kchunks;
    const int nsub = nsteps * 3;
    const uint4* wblk = (const uint4*)a.wpk + (size_t)nb * nsub * B_CH;

    uint4 ra[A_IT];
    uint4 rb[B_IT];

    auto fetch_a = [&](int step) {
        const int ta = step / a.kchunks, kc = step - ta * a.kchunks;
        const uint16_t* fp = zframe(a.z, t + ta);
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            const int idx = tid + NT * it;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (idx < A_CH) {
                const int pix = idx >> 2, gg = idx & 3;
                const int r = pix / LW, c = pix - r * LW;
                const int gy = i0 + r - 1, gx = j0 + c - 1;
                const int ch = kc * 32 + gg * 8;
                if (fp && gy >= 0 && gy < a.h_in && gx >= 0 && gx < a.w_in && ch < a.cin)
                    v = *(const uint4*)(fp + ((int64_t)gy * a.w_in + gx) * a.cin + ch);
            }
            ra[it] = v;
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            const int idx = tid + NT * it;
            if (idx < A_CH) {
                const int pix = idx >> 2, gg = idx & 3;
                lds_a[buf][pix * 4 + (gg ^ swz(pix))] = ra[it];
            }
        }
    };
    auto fetch_b = [&](int sub) {
        const uint4* src = wblk + (size_t)sub * B_CH;
#pragma unroll
        for (int it = 0; it < B_IT; ++it) {
            const int idx = tid + NT * it;
            rb[it] = idx < B_CH ? src[idx] : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_b = [&](int buf) {
#pragma unroll
        for (int it = 0; it < B_IT; ++it) {
            const int idx = tid + NT * it;
            if (idx < B_CH) lds_b[buf][idx] = rb[it];
        }
    };
    auto a_frag = [&](int buf, int ly, int lx) -> bf16x8 {
        const int pix = ly * LW + lx;
        return as_bf16x8(lds_a[buf][pix * 4 + (g ^ swz(pix))]);
    };

    // prologue: step 0's tile and sub-step 0's weights
    fetch_a(0);
    fetch_b(0);
    store_a(0);
    store_b(0);
    __syncthreads();

    for (int sub = 0; sub < nsub; ++sub) {
        const int step = sub / 3, d = sub - step * 3;
        const int abuf = step & 1, bbuf = sub & 1;
        const bool more_b = sub + 1 < nsub;
        const bool more_a = step + 1 < nsteps;
        if (more_b) fetch_b(sub + 1);
        if (more_a && d == 0) fetch_a(step + 1);  // lands in LDS after sub-step d == 2

        // B fragments of taps (b, d), b = 0..2, for this wave's channels
        bf16x8 bq[3][NFW];
#pragma unroll
        for (int b = 0; b < 3; ++b)
#pragma unroll
            for (int f = 0; f < NFW; ++f) {
                const int nl = 16 * (wn * NFW + f) + k16;
                bq[b][f] = as_bf16x8(lds_b[bbuf][(b * NTILE + nl) * 4 + (g ^ swz(nl))]);
            }

        if (UP == 1) {
            // LDS row s holds source row i0 + s - 1; output row r reads rows r+b.
#pragma unroll
            for (int s = 0; s < G::TS_H + 2; ++s) {
                const bf16x8 av = a_frag(abuf, s, 16 * wm + k16 + d);
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const int r = s - b;
                    if (r >= 0 && r < G::TS_H) {
#pragma unroll
                        for (int f = 0; f < NFW; ++f)
                            acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[b][f], acc[r][f], 0, 0, 0);
                    }
                }
            }
        } else {
            // M fragment m = rr*4 + p*2 + q: source row 2*wm + rr, phase (p, q).
            // Column offsets used by this d: q=0 -> floor((d-1)/2), q=1 -> floor(d/2).
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
                for (int oy = -1; oy <= 1; ++oy) {
                    const int ly = 2 * wm + rr + oy + 1;
                    const int ox0 = (d - 1) >> 1;  // q = 0
                    const int ox1 = d >> 1;        // q = 1
                    const bf16x8 a0 = a_frag(abuf, ly, k16 + ox0 + 1);
                    const bf16x8 a1 = (ox1 == ox0) ? a0 : a_frag(abuf, ly, k16 + ox1 + 1);
#pragma unroll
                    for (int p = 0; p < 2; ++p)
#pragma unroll
                        for (int b = 0; b < 3; ++b) {
                            if (((p + b - 1) >> 1) != oy) continue;
#pragma unroll
                            for (int f = 0; f < NFW; ++f) {
                                acc[rr * 4 + p * 2 + 0][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    a0, bq[b][f], acc[rr * 4 + p * 2 + 0][f], 0, 0, 0);
                                acc[rr * 4 + p * 2 + 1][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    a1, bq[b][f], acc[rr * 4 + p * 2 + 1][f], 0, 0, 0);
                            }
                        }
                }
            }
        }

        if (more_b) store_b(bbuf ^ 1);
        if (more_a && d == 2) store_a(abuf ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // v = acc + bias (+ res), rounded to bf16 and stored.  act = SiLU(RMSNorm(v))
    // from the rounded value: the channel sum of squares is reduced over the 16
    // lanes that hold one pixel, then over the WN waves through LDS (the main
    // loop's last barrier has retired every read of lds_a).
    const int n0 = nb * NTILE + wn * NFW * 16;
    uint16_t* out = (uint16_t*)a.out;
    uint16_t* act = (uint16_t*)a.act_out;
    const uint16_t* res = (const uint16_t*)a.res;
    float* red = (float*)&lds_a[0][0];  // [WN][4 M-waves][MF][16 pixels]

    auto pixel_of = [&](int m, int i, int& y, int& x) {
        const int k = 4 * g + i;  // pixel within the 16-pixel fragment
        if (UP == 1) {
            y = i0 + m;
            x = j0 + 16 * wm + k;
        } else {
            const int rr = m >> 2, p = (m >> 1) & 1, q = m & 1;
            y = 2 * (i0 + 2 * wm + rr) + p;
            x = 2 * (j0 + k) + q;
        }
    };
    auto value = [&](int m, int i, int f, int64_t pbase, bool valid) -> float {
        const int n = n0 + 16 * f + k16;
        if (n >= a.cout) return 0.f;
        float v = acc[m][f][i];
        if (a.bias) v += a.bias[n];
        if (res && valid) v += bf2f(res[pbase + n]);
        return bf2f(f2bf(v));
    };

    // pass 1: store v; per-pixel partial sums of squares for the act
#pragma clang loop unroll(full)
    for (int m = 0; m < MF; ++m) {
#pragma clang loop unroll(full)
        for (int i = 0; i < 4; ++i) {
            int y, x;
            pixel_of(m, i, y, x);
            const bool valid = y < a.h_out && x < a.w_out;
            const int64_t pbase = (((int64_t)t * a.h_out + y) * a.w_out + x) * a.cout;
            float ss = 0.f;
#pragma unroll
            for (int f = 0; f < NFW; ++f) {
                const float v = value(m, i, f, pbase, valid);
                const int n = n0 + 16 * f + k16;
                if (out && valid && n < a.cout) out[pbase + n] = f2bf(v);
                ss += v * v;
            }
            if (act) {
                ss += __shfl_xor(ss, 1, 64);
                ss += __shfl_xor(ss, 2, 64);
                ss += __shfl_xor(ss, 4, 64);
                ss += __shfl_xor(ss, 8, 64);
                if (k16 == 0) red[((wn * 4 + wm) * MF + m) * 16 + 4 * g + i] = ss;
            }
        }
    }
    if (!act) return;
    __syncthreads();
    // pass 2: the act from the full channel sum
#pragma clang loop unroll(full)
    for (int m = 0; m < MF; ++m) {
#pragma clang loop unroll(full)
        for (int i = 0; i < 4; ++i) {
            int y, x;
            pixel_of(m, i, y, x);
            const bool valid = y < a.h_out && x < a.w_out;
            const int64_t pbase = (((int64_t)t * a.h_out + y) * a.w_out + x) * a.cout;
            float ss = 0.f;
#pragma unroll
            for (int h = 0; h < WN; ++h) ss += red[((h * 4 + wm) * MF + m) * 16 + 4 * g + i];
            const float inv = 1.0f / sqrtf(ss / (float)a.cout + a.eps);
#pragma unroll
            for (int f = 0; f < NFW; ++f) {
                const int n = n0 + 16 * f + k16;
                if (n < a.cout && valid) {
                    const float zz = a.gamma[n] * value(m, i, f, pbase, valid) * inv;
                    act[pbase + n] = f2bf(zz / (1.0f + expf(-zz)));
                }
            }
        }
    }
}

template <int UP, int NF, int WN>
hipError_t launch_v2(const ConvArgs& a, hipStream_t s)
{
    using G = Geo<UP>;
    const int tiles = ((a.h_in + G::TS_H - 1) / G::TS_H) * ((a.w_in + G::TS_W - 1) / G::TS_W);
    const int64_t total = (int64_t)tiles * a.t_out * a.nblocks;
    if (total <= 0 || total > (int64_t)0x7fffffff - 8) return hipErrorInvalidValue;
    const int64_t grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((conv3_v2_kernel<UP, NF, WN>), dim3((unsigned)grid), dim3(256 * WN), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool v2_conv_applies(int ntile, int kh, int kw, int up_s)
{
    return kh == 3 && kw == 3 && (up_s == 1 || up_s == 2) && (ntile == 96 || ntile == 128);
}

hipError_t launch_conv_bf16_v2(const ConvArgs& a, hipStream_t s)
{
    if (!v2_conv_applies(a.ntile, a.kh, a.kw, a.up_s)) return hipErrorInvalidValue;
    if (a.up_s == 1) return a.ntile == 96 ? launch_v2<1, 6, 2>(a, s) : launch_v2<1, 8, 2>(a, s);
    return a.ntile == 96 ? launch_v2<2, 6, 2>(a, s) : launch_v2<2, 8, 2>(a, s);
}

}  // namespace cc3d
