// bf16 causal conv3d as an implicit GEMM on gfx950 MFMA (v_mfma_f32_16x16x32_bf16).
//
// GEMM view: M = output pixels of one frame, N = output channels, K = Cin x taps.
// A workgroup (4 waves, 256 threads) owns one output frame, one block of NTILE
// output channels and a TS_H x TS_W tile of *source* pixels (the conv input before
// the nearest upsample).  K is walked in steps of (temporal tap, 32 channels):
//   1. the source tile plus a one-pixel border, 32 channels deep, is staged in LDS
//      (zero outside the image, for zero history frames and past Cin);
//   2. the packed weights of that step (all spatial taps, NTILE channels) are
//      staged in LDS;
//   3. each wave runs kh*kw spatial taps of MFMAs, reading A fragments straight
//      out of the source tile.
// The nearest 2x spatial upsample is never materialised: with up_s = 2 an M
// fragment is 16 source columns of one source row at one output phase (p, q),
// i.e. output pixels (2i+p, 2j+q); spatial tap (b, d) of that phase reads source
// offset (floor((p+b-1)/2), floor((q+d-1)/2)).  Zero padding of the upsampled
// image is exactly "source pixel outside the image".  The temporal growth and the
// causal history are resolved per frame by the ZWindow map.
//
// Strided convs (DOWN = 2, the encoder side): the tile is TS_H x TS_W *output*
// pixels, which read input rows 2y-1 .. 2y+1 and columns 2x-1 .. 2x+1; the LDS
// tile keeps the even input columns first and the odd ones after them, so the
// 16 output columns of a fragment read 16 consecutive LDS pixels at every column
// tap (columns 2x + d: even half at x + d/2 for d = 0, 2, odd half at x for
// d = 1), as the unstrided reads do.  A temporal stride maps output frame t to
// window frames t_stride*t + t_first + (0 .. kt-1).
//
// Epilogue (fp32): + bias, + residual, round to bf16 and store (or store the
// 8-bit code of the fp32 result, see rgb8_code); optionally the
// channel RMSNorm + SiLU of the stored value, reduced across the 16 lanes that
// hold one pixel's channels (only when one workgroup holds every channel).
//
// MFMA operand layout (16x16x32): lane l supplies row (l & 15) of A / column
// (l & 15) of B with 8 consecutive K values from K group (l >> 4); the result
// lane l holds rows 4*(l >> 4) + i, column (l & 15).
#include <cstdlib>

#include "cc3d_device.h"

namespace cc3d {
namespace {

template <int UP, int DOWN, int KS, int NF, int TS_H, int SW>
__global__ __launch_bounds__(256) void conv_bf16_kernel(ConvArgs a)
{
    static_assert(UP == 1 || DOWN == 1, "a conv either upsamples or strides");
    constexpr int HALO = (KS - 1) / 2;
    constexpr int TS_W = 16 * SW;
    // LDS tile: the input rows and columns the tile's outputs read
    constexpr int LH = DOWN * (TS_H - 1) + 2 * HALO + 1, LW = DOWN * (TS_W - 1) + 2 * HALO + 1;
    constexpr int NE = (LW + 1) / 2;  // DOWN = 2: even input columns, stored first
    constexpr int NPH = UP * UP;
    constexpr int NTILE = 16 * NF;
    constexpr int TAPS = KS * KS;
    constexpr int RPW = TS_H / 4;  // source rows per wave
    constexpr int MF = RPW * SW * NPH;
    constexpr int A_CHUNKS = LH * LW * 4;
    constexpr int B_CHUNKS = TAPS * NTILE * 4;
    static_assert(TS_H % 4 == 0, "four waves split the tile rows");

    __shared__ uint4 lds_a[A_CHUNKS];
    __shared__ uint4 lds_b[B_CHUNKS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, k16 = lane & 15;
    // tiles cover the source frame (UP = 2) or the output frame (strided or not)
    const int tiles_w = ((UP == 2 ? a.w_in : a.w_out) + TS_W - 1) / TS_W;
    const int i0 = (blockIdx.x / tiles_w) * TS_H;
    const int j0 = (blockIdx.x % tiles_w) * TS_W;
    const int nb = blockIdx.y;
    const int t = blockIdx.z;

    f32x4 acc[MF][NF];
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = a.kt * a.kchunks;
    const uint4* wblk = (const uint4*)a.wpk + (size_t)nb * nsteps * B_CHUNKS;

    for (int step = 0; step < nsteps; ++step) {
        const int ta = step / a.kchunks, kc = step - ta * a.kchunks;
        const uint16_t* fp = zframe(a.z, a.t_stride * t + a.t_first + ta);
        __syncthreads();  // every wave is done reading the previous step
        for (int idx = tid; idx < A_CHUNKS; idx += 256) {
            const int pix = idx >> 2, gg = idx & 3;
            const int r = pix / LW, lc = pix - r * LW;
            const int c = DOWN == 1 ? lc : (lc < NE ? 2 * lc : 2 * (lc - NE) + 1);  // input column in the tile
            const int gy = DOWN * i0 + r - HALO, gx = DOWN * j0 + c - HALO;
            const int ch = kc * 32 + gg * 8;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (fp && gy >= 0 && gy < a.h_in && gx >= 0 && gx < a.w_in && ch < a.cin)
                v = *(const uint4*)(fp + ((int64_t)gy * a.w_in + gx) * a.cin + ch);
            lds_a[pix * 4 + (gg ^ swz(pix))] = v;
        }
        const uint4* bsrc = wblk + (size_t)step * B_CHUNKS;
        for (int idx = tid; idx < B_CHUNKS; idx += 256) lds_b[idx] = bsrc[idx];
        __syncthreads();

#pragma unroll
        for (int tb = 0; tb < KS; ++tb) {
#pragma unroll
            for (int td = 0; td < KS; ++td) {
                bf16x8 bfr[NF];
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const int nl = 16 * f + k16;
                    bfr[f] = as_bf16x8(lds_b[((tb * KS + td) * NTILE + nl) * 4 + (g ^ swz(nl))]);
                }
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    const int ph = m % NPH;
                    const int s = (m / NPH) % SW;
                    const int r = wave * RPW + m / (NPH * SW);
                    int ly, lx;
                    if (UP == 1 && DOWN == 1) {
                        ly = r + tb;
                        lx = 16 * s + k16 + td;
                    } else if (DOWN == 2) {
                        ly = 2 * r + tb;
                        lx = (td & 1) ? NE + 16 * s + k16 + (td >> 1) : 16 * s + k16 + (td >> 1);
                    } else {
                        const int oy = ((ph >> 1) + tb - HALO) >> 1;  // floor((p + dy) / 2)
                        const int ox = ((ph & 1) + td - HALO) >> 1;
                        ly = r + oy + HALO;
                        lx = 16 * s + k16 + ox + HALO;
                    }
                    const int pix = ly * LW + lx;
                    const bf16x8 av = as_bf16x8(lds_a[pix * 4 + (g ^ swz(pix))]);
#pragma unroll
                    for (int f = 0; f < NF; ++f)
                        acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bfr[f], acc[m][f], 0, 0, 0);
                }
            }
        }
    }

    // ---------------------------------------------------------------- epilogue
    const int n0 = nb * NTILE;
    uint16_t* out = (uint16_t*)a.out;
    uint16_t* act = (uint16_t*)a.act_out;
    const uint16_t* res = (const uint16_t*)a.res;
#pragma unroll
    for (int m = 0; m < MF; ++m) {
        const int ph = m % NPH;
        const int s = (m / NPH) % SW;
        const int r = wave * RPW + m / (NPH * SW);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 4 * g + i;  // pixel within the 16-pixel fragment
            int y, x;
            if (UP == 1) {
                y = i0 + r;
                x = j0 + 16 * s + k;
            } else {
                y = 2 * (i0 + r) + (ph >> 1);
                x = 2 * (j0 + 16 * s + k) + (ph & 1);
            }
            const bool valid = y < a.h_out && x < a.w_out;
            const int64_t pbase = (((int64_t)t * a.h_out + y) * a.w_out + x) * a.cout;
            float vr[NF];
            float ss = 0.f;
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int n = n0 + 16 * f + k16;
                float v = 0.f;
                if (n < a.cout) {
                    v = acc[m][f][i];
                    if (a.bias) v += a.bias[n];
                    if (res && valid) v += bf2f(res[pbase + n]);
                    if (a.out_u8 && out && valid) ((uint8_t*)out)[pbase + n] = rgb8_code(v);
                    const uint16_t hb = f2bf(v);
                    v = bf2f(hb);
                    if (out && valid && !a.out_u8) out[pbase + n] = hb;
                }
                vr[f] = v;
                ss += v * v;
            }
            if (act) {
                ss += __shfl_xor(ss, 1, 64);
                ss += __shfl_xor(ss, 2, 64);
                ss += __shfl_xor(ss, 4, 64);
                ss += __shfl_xor(ss, 8, 64);
                const float inv = 1.0f / sqrtf(ss / (float)a.cout + a.eps);
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const int n = n0 + 16 * f + k16;
                    if (n < a.cout && valid) {
                        const float zz = a.gamma[n] * vr[f] * inv;
                        act[pbase + n] = f2bf(zz / (1.0f + expf(-zz)));
                    }
                }
            }
        }
    }
}

template <int UP, int DOWN, int KS, int NF>
hipError_t launch_cfg(const ConvArgs& a, hipStream_t s)
{
    constexpr int TS_H = (UP == 2) ? 4 : 16;
    constexpr int SW = 1;
    const int th = UP == 2 ? a.h_in : a.h_out, tw = UP == 2 ? a.w_in : a.w_out;
    const int tiles = ((th + TS_H - 1) / TS_H) * ((tw + 16 * SW - 1) / (16 * SW));
    dim3 grid(tiles, a.nblocks, a.t_out);
    hipLaunchKernelGGL((conv_bf16_kernel<UP, DOWN, KS, NF, TS_H, SW>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int UP, int DOWN, int KS>
hipError_t launch_nf(const ConvArgs& a, hipStream_t s)
{
    switch (a.ntile) {
    case 16: return launch_cfg<UP, DOWN, KS, 1>(a, s);
    case 32: return launch_cfg<UP, DOWN, KS, 2>(a, s);
    case 64: return launch_cfg<UP, DOWN, KS, 4>(a, s);
    case 96: return launch_cfg<UP, DOWN, KS, 6>(a, s);
    case 128: return launch_cfg<UP, DOWN, KS, 8>(a, s);
    default: return hipErrorInvalidValue;
    }
}

// Packed layout per (channel block, temporal tap, 32-channel chunk): the
// kh*kw spatial taps, each NTILE rows of 32 channels with the 16-byte chunks
// swizzled as in LDS.  Spatial taps are ordered row-major (b, d), or column
// major (d, b) for the v2 kernels, whose sub-steps take one column tap at a time.
// tfold (8 input channels, family 6): one K step whose 8-channel group g holds
// temporal tap g (K index 8 g + c = tap g, channel c; the fourth group zeros).
__global__ void pack_bf16_kernel(const uint16_t* w, uint16_t* wpk, int cout, int cin, int kt,
                                 int kh, int kw, int ntile, int nblocks, int kchunks, int dmajor, int tfold)
{
    const int taps = kh * kw;
    const int kt_steps = tfold ? 1 : kt;
    const int64_t total = (int64_t)nblocks * kt_steps * kchunks * taps * ntile * 32;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int e = (int)(idx & 31);
        int64_t row = idx >> 5;
        const int nl = (int)(row % ntile);
        row /= ntile;
        const int tap = (int)(row % taps);
        row /= taps;
        const int kc = (int)(row % kchunks);
        row /= kchunks;
        int ta = (int)(row % kt_steps);
        const int nb = (int)(row / kt_steps);
        const int gphys = e >> 3, el = e & 7;
        const int glog = gphys ^ swz(nl);
        const int n = nb * ntile + nl;
        int c = kc * 32 + glog * 8 + el;
        if (tfold) {
            ta = glog;
            c = el;
        }
        const int b = dmajor ? tap % kh : tap / kw;
        const int d = dmajor ? tap / kh : tap % kw;
        uint16_t v = 0;
        if (n < cout && c < cin && ta < kt) v = w[((((int64_t)n * cin + c) * kt + ta) * kh + b) * kw + d];
        wpk[idx] = v;
    }
}

}  // namespace

bool bf16_conv_supported(int cout, int kh, int kw, int up_s)
{
    if (kh != kw || (kh != 1 && kh != 3)) return false;
    if (up_s != 1 && up_s != 2) return false;
    int nt, nb;
    bf16_conv_tiling(cout, &nt, &nb);
    return nt > 0;
}

void bf16_conv_tiling(int cout, int* ntile, int* nblocks)
{
    int nt = 0;
    if (cout <= 16) nt = 16;
    else if (cout <= 32) nt = 32;
    else if (cout <= 64) nt = 64;
    else if (cout <= 96) nt = 96;
    else if (cout <= 128) nt = 128;
    else if (cout % 96 == 0) nt = 96;
    else if (cout % 128 == 0) nt = 128;
    else nt = 64;
    *ntile = nt;
    *nblocks = nt ? (cout + nt - 1) / nt : 0;
}

int bf16_conv_family(int cout, int cin, int kt, int kh, int kw, int up_s, int plain, int fold)
{
    const char* e = getenv("CC3D_CONV_FAMILY");
    if (e && atoi(e) == 1) return 1;
    if (head_conv_applies(cout, cin, kt, kh, kw, up_s)) return 3;
    if (plain && pw_conv_applies(cout, kh, kw, up_s)) return 4;
    int nt, nb;
    bf16_conv_tiling(cout, &nt, &nb);
    if (fold && phase_conv_applies(nt, kh, kw, up_s)) return 5;
    return v2_conv_applies(nt, kh, kw, up_s) ? 2 : 1;
}

size_t bf16_packed_elems(int cout, int cin, int kt, int kh, int kw, int family)
{
    if (family == 3) return head_packed_elems(cin);
    if (family == 4) return pw_packed_elems(cout, cin, kt);
    if (family == 5) return phase_packed_elems(cout, cin, kt);
    int nt, nb;
    bf16_conv_tiling(cout, &nt, &nb);
    if (family == 7) {  // the strided tile in 192-channel blocks
        nt = 192;
        nb = (cout + 191) / 192;
    }
    const int kchunks = (cin + 31) / 32;
    return (size_t)nb * (family == 6 ? 1 : kt) * kchunks * kh * kw * nt * 32;
}

hipError_t launch_pack_bf16(const void* w, void* wpk, int cout, int cin, int kt, int kh, int kw,
                            int family, hipStream_t s)
{
    if (family == 3) return launch_pack_head(w, wpk, cout, cin, s);
    if (family == 4) return launch_pack_pw(w, wpk, cout, cin, kt, s);
    if (family == 5) return launch_pack_phase(w, wpk, cout, cin, kt, s);
    int nt, nb;
    bf16_conv_tiling(cout, &nt, &nb);
    if (family == 7) {
        nt = 192;
        nb = (cout + 191) / 192;
    }
    const int kchunks = (cin + 31) / 32;
    const size_t total = bf16_packed_elems(cout, cin, kt, kh, kw, family);
    int blocks = (int)((total + 255) / 256);
    if (blocks > 65536) blocks = 65536;
    const int dmajor = (family == 2 || family == 6 || family == 7) ? 1 : 0;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t*)w,
                       (uint16_t*)wpk, cout, cin, kt, kh, kw, nt, nb, kchunks, dmajor, family == 6 ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_conv_bf16(const ConvArgs& a, hipStream_t s)
{
    if (a.kh != a.kw) return hipErrorInvalidValue;
    if (a.family == 3) return launch_conv_head(a, s);
    if (a.family == 4) return launch_conv_pw(a, s);
    if (a.family == 5) return launch_conv_phase(a, s);
    if (a.family == 2 || a.family == 6 || a.family == 7) return launch_conv_bf16_v2(a, s);
    if (a.t_stride < 1 || a.t_stride > 2 || (a.down_s != 1 && a.down_s != 2) || (a.down_s == 2 && a.up_s != 1))
        return hipErrorInvalidValue;
    if (a.down_s == 2) return a.kh == 3 ? launch_nf<1, 2, 3>(a, s) : launch_nf<1, 2, 1>(a, s);
    if (a.up_s == 1 && a.kh == 3) return launch_nf<1, 1, 3>(a, s);
    if (a.up_s == 2 && a.kh == 3) return launch_nf<2, 1, 3>(a, s);
    if (a.up_s == 1 && a.kh == 1) return launch_nf<1, 1, 1>(a, s);
    if (a.up_s == 2 && a.kh == 1) return launch_nf<2, 1, 1>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace cc3d
