// Output-head conv on gfx950 MFMA: a 3x3x3 causal conv to at most three
// channels (RGB), on a nearest-2x upsampled input (UP = 2) or at the input's own
// size (UP = 1).
//
// With three output channels, the GEMM view of the other kernels (N = output
// channels) leaves 13 of 16 MFMA columns idle.  Here the spatial taps go into N
// and the temporal taps into K: for output frame t, every source pixel s and
// every spatial tap (b, d) and channel o,
//
//     P[s][(b, d, o)] = sum_{a, c} X[t + a][s][c] * W[o][c][a][b][d]
//
// is one GEMM with M = source pixels, K = 3 window frames x Cin, N = 9 spatial
// taps x 3 channels (27, padded to 32).  An output pixel (y, x) of frame t then
// sums, for each spatial tap, one entry of P: with UP = 2, tap (b, d) of output
// phase (p, q) = (y & 1, x & 1) reads source (y/2 + floor((p+b-1)/2), x/2 +
// floor((q+d-1)/2)) -- nearest upsampling followed by zero padding of the
// upsampled image is exactly "zero outside the source image"; with UP = 1 it
// reads (y + b - 1, x + d - 1).  Window frame t + a of the causal window is the
// temporal tap a.  Every product of the conv's definition is formed once (in
// the MFMA) and every sum is taken in fp32, in a different order from the direct
// form; no weights are pre-summed.
//
// A workgroup owns a tile of 8 x 16 source pixels (16 x 32 output pixels, or
// 8 x 16 with UP = 1) and a run of consecutive output frames.  Each window frame
// of the run is loaded once: its tile plus a one-pixel border (18 x 10 pixels,
// 12 M fragments) goes straight into MFMA operand registers, into a ring of
// three frames (output frame t reads frames t, t+1, t+2; frame t+3 replaces
// frame t as soon as t's products are formed).  P goes to one of two LDS
// buffers: a thread gathers output frame t's taps from one buffer, then forms
// the products of frame t+1 and writes them to the other; one barrier per
// frame.
#include "cc3d_device.h"

namespace cc3d {
namespace {

constexpr int TH = 8, TW = 16;                  // source tile
constexpr int BH = TH + 2, BW = TW + 2;         // with the one-pixel border
constexpr int BPIX = BH * BW;                   // 180
constexpr int MFR = (BPIX + 15) / 16;           // 12 M fragments of 16 pixels
constexpr int MFW = MFR / 4;                    // 3 per wave
constexpr int NFR = 2;                          // N = 32: column n = 9 b + 3 d + o (27 used)
constexpr int PSTR = 33;                        // floats per pixel in the P table (odd: see below)
constexpr int PBUF = MFR * 16 * PSTR;           // floats per P buffer

// P table position of column n of bordered-tile pixel L.  An odd pixel stride
// puts the same column of 16 neighbouring pixels in 16 different banks, and the
// position stays a base plus a constant (one address register per pixel).
__device__ __forceinline__ int pidx(int L, int n) { return L * PSTR + n; }

template <int UP, int KC>
__global__ __launch_bounds__(256, 2) void conv_head_kernel(ConvArgs a, int fpw)
{
    __shared__ float ptab[2 * PBUF];

    const int tiles_w = (a.w_in + TW - 1) / TW;
    const int tiles_h = (a.h_in + TH - 1) / TH;
    const int ntiles = tiles_w * tiles_h;
    const int tgroups = (a.t_out + fpw - 1) / fpw;
    // work items (tile, time group), dealt to the 8 XCDs in contiguous ranges
    const int total = ntiles * tgroups;
    const int per_xcd = (total + 7) >> 3;
    const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (w >= total) return;
    const int tg = w % tgroups, tile = w / tgroups;
    // tiles in strips of four tile rows, walked column by column (row fastest):
    // the tiles above and below, and the ones beside, run close in time and
    // share their border rows and columns in L2
    constexpr int SR = 4;
    const int strip = tile / (SR * tiles_w), k = tile - strip * SR * tiles_w;
    const int sr = min(SR, tiles_h - strip * SR);
    const int i0 = (strip * SR + k % sr) * TH, j0 = (k / sr) * TW;
    const int t0 = tg * fpw;
    const int t1 = min(t0 + fpw, a.t_out);
    const int z1 = t1 + 2;  // window frames t0 .. z1-1 are read

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, k16 = lane & 15;

    // weights (MFMA row operand): temporal tap ta, row 16 f + k16, channels
    // 32 kc + 8 g .. + 7
    bf16x8 wa[3][KC][NFR];
    const uint4* wp = (const uint4*)a.wpk;
#pragma unroll
    for (int ta = 0; ta < 3; ++ta)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int f = 0; f < NFR; ++f)
                wa[ta][kc][f] = __builtin_bit_cast(bf16x8, wp[((ta * KC + kc) * NFR + f) * 64 + lane]);

    // this lane's pixel in each of the wave's M fragments: byte offset inside a
    // frame of its 8-channel group, OOB outside the image (loads return zeros)
    uint32_t poff[MFW];
#pragma unroll
    for (int mm = 0; mm < MFW; ++mm) {
        const int L = (wave * MFW + mm) * 16 + k16;
        const int r = L / BW, c = L - r * BW;
        const int gy = i0 + r - 1, gx = j0 + c - 1;
        poff[mm] = (L < BPIX && gy >= 0 && gy < a.h_in && gx >= 0 && gx < a.w_in)
                       ? (uint32_t)(((gy * a.w_in + gx) * a.cin + g * 8) * 2)
                       : OOB;
    }
    const uint32_t frame_bytes = (uint32_t)(a.z.frame_elems * 2);
    bf16x8 xb[3][KC][MFW];
    auto load_frame = [&](const int zi, const int slot) {
        const uint16_t* fp = zframe(a.z, zi);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(fp, fp ? frame_bytes : 0u);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int mm = 0; mm < MFW; ++mm)
                xb[slot][kc][mm] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(poff[mm] + (uint32_t)(kc * 64)), 0, 0));
    };

    // P of one output frame whose window frame t sits in ring slot s0
    f32x4 acc[MFW][NFR];
    auto products = [&](const int s0) {
#pragma unroll
        for (int mm = 0; mm < MFW; ++mm)
#pragma unroll
            for (int f = 0; f < NFR; ++f) acc[mm][f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ta = 0; ta < 3; ++ta)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                for (int mm = 0; mm < MFW; ++mm)
#pragma unroll
                    for (int f = 0; f < NFR; ++f)
                        acc[mm][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ta][kc][f], xb[(s0 + ta) % 3][kc][mm],
                                                                             acc[mm][f], 0, 0, 0);
    };
    // acc[mm][f] = D[n][pixel]: lane (g, k16) holds n = 16 f + 4 g .. + 3 of pixel k16
    auto write_p = [&](float* pb) {
#pragma unroll
        for (int mm = 0; mm < MFW; ++mm) {
            const int L = (wave * MFW + mm) * 16 + k16;
#pragma unroll
            for (int f = 0; f < NFR; ++f)
#pragma unroll
                for (int j = 0; j < 4; ++j) pb[pidx(L, 16 * f + 4 * g + j)] = acc[mm][f][j];
        }
    };

    const int cout = a.cout;
    float bias[3];
#pragma unroll
    for (int o = 0; o < 3; ++o) bias[o] = (a.bias && o < cout) ? a.bias[o] : 0.f;

    // UP = 2: the two output pixels of this thread are row oy, columns 2 sj and
    // 2 sj + 1 of the 16 x 32 output tile (source row si, phase p = oy & 1).
    // UP = 1: threads 0..127 own output pixel (si, sj) of the 8 x 16 tile.
    constexpr int NQ = UP;
    const int oy = tid >> 4, sj = tid & 15;
    const int p = oy & 1, si = UP == 2 ? oy >> 1 : oy;
    const int Y = UP == 2 ? 2 * i0 + oy : i0 + oy, X = UP == 2 ? 2 * (j0 + sj) : j0 + sj;
    const bool mine = Y < a.h_out && X < a.w_out && (UP == 2 || tid < TH * TW);

    // gather: UP = 2: tap (b, d) of output pixel (oy, 2 sj + q) reads
    // bordered-tile pixel (si + 1 + floor((p+b-1)/2), sj + 1 + floor((q+d-1)/2)):
    //   q = 0: d = 0 -> column sj, d = 1, 2 -> sj + 1;  q = 1: d = 0, 1 -> sj + 1, d = 2 -> sj + 2.
    // UP = 1: tap (b, d) of output pixel (si, sj) reads (si + b, sj + d).
    auto gather_store = [&](const float* pb, const int t) {
        if (!mine) return;
        float v[NQ][3];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int o = 0; o < 3; ++o) v[q][o] = bias[o];
#pragma unroll
        for (int b = 0; b < 3; ++b) {
            const int row = UP == 2 ? si + 1 + ((p + b - 1) >> 1) : si + b;
            const int L0 = row * BW + sj;
#pragma unroll
            for (int o = 0; o < 3; ++o) {
                if (UP == 2) {
                    const float c1 = pb[pidx(L0 + 1, 9 * b + 3 + o)];
                    v[0][o] += pb[pidx(L0, 9 * b + o)] + c1 + pb[pidx(L0 + 1, 9 * b + 6 + o)];
                    v[NQ - 1][o] += pb[pidx(L0 + 1, 9 * b + o)] + c1 + pb[pidx(L0 + 2, 9 * b + 6 + o)];
                } else {
                    v[0][o] += pb[pidx(L0, 9 * b + o)] + pb[pidx(L0 + 1, 9 * b + 3 + o)] +
                               pb[pidx(L0 + 2, 9 * b + 6 + o)];
                }
            }
        }
        const int64_t base = (((int64_t)t * a.h_out + Y) * a.w_out + X) * cout;
        const uint16_t* res = (const uint16_t*)a.res;
        if (res) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int o = 0; o < 3; ++o)
                    if (o < cout && X + q < a.w_out) v[q][o] += bf2f(res[base + q * cout + o]);
        }
        if (UP == 2 && cout == 3) {
            // 6 values of two neighbouring pixels, from an even element (X and
            // w_out are even): three 4-byte (bf16) or 2-byte (8-bit) stores
            if (a.out_u8) {
                uint16_t* o8 = (uint16_t*)((uint8_t*)a.out + base);
                o8[0] = (uint16_t)(rgb8_code(v[0][0]) | (rgb8_code(v[0][1]) << 8));
                o8[1] = (uint16_t)(rgb8_code(v[0][2]) | (rgb8_code(v[NQ - 1][0]) << 8));
                o8[2] = (uint16_t)(rgb8_code(v[NQ - 1][1]) | (rgb8_code(v[NQ - 1][2]) << 8));
            } else {
                uint32_t* o32 = (uint32_t*)((uint16_t*)a.out + base);
                o32[0] = pack_bf16x2(v[0][0], v[0][1]);
                o32[1] = pack_bf16x2(v[0][2], v[NQ - 1][0]);
                o32[2] = pack_bf16x2(v[NQ - 1][1], v[NQ - 1][2]);
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (X + q >= a.w_out) continue;
#pragma unroll
            for (int o = 0; o < 3; ++o) {
                if (o >= cout) continue;
                if (a.out_u8)
                    ((uint8_t*)a.out)[base + q * cout + o] = rgb8_code(v[q][o]);
                else
                    ((uint16_t*)a.out)[base + q * cout + o] = f2bf(v[q][o]);
            }
        }
    };

    // Output frame t (ring slot of its first window frame: PH = (t - t0) mod 3).
    // On entry P of frame t is being written to buffer (t - t0) & 1.  The two
    // waves of each SIMD (two workgroups per CU) overlap one's gather with the
    // other's MFMAs; within a wave the gather comes first, so the accumulators
    // are not live beside the gathered values.
    auto step = [&](const int t, const int PH) {
        float* pb = ptab + ((t - t0) & 1) * PBUF;
        float* pn = ptab + ((t + 1 - t0) & 1) * PBUF;
        __syncthreads();  // P of frame t is complete; every gather of frame t-1 is done
        gather_store(pb, t);
        if (t + 1 < t1) {
            products((PH + 1) % 3);                           // frame t+1: window t+1 .. t+3
            if (t + 4 < z1) load_frame(t + 4, (PH + 1) % 3);  // replaces window frame t+1
            write_p(pn);
        }
    };

    load_frame(t0, 0);
    load_frame(t0 + 1, 1);
    load_frame(t0 + 2, 2);
    products(0);
    if (t0 + 3 < z1) load_frame(t0 + 3, 0);
    write_p(ptab);
    for (int tb = t0; tb < t1; tb += 3) {
        step(tb, 0);
        if (tb + 1 < t1) step(tb + 1, 1);
        if (tb + 2 < t1) step(tb + 2, 2);
    }
}

}  // namespace

bool head_conv_applies(int cout, int cin, int kt, int kh, int kw, int up_s)
{
    return cout >= 1 && cout <= 3 && kt == 3 && kh == 3 && kw == 3 && (up_s == 1 || up_s == 2) && cin % 32 == 0 &&
           cin >= 32 && cin <= 96;
}

size_t head_packed_elems(int cin)
{
    return (size_t)3 * (cin / 32) * NFR * 64 * 8;
}

namespace {
// Packed head weights: for each (temporal tap a, 32-channel chunk kc, N
// fragment f), 64 lanes of 8 channels: lane (g, k16) holds
// W[o][32 kc + 8 g + e][a][b][d] for row n = 16 f + k16 = 9 b + 3 d + o (zero for
// n >= 27 or o >= cout).
__global__ void pack_head_kernel(const uint16_t* w, uint16_t* wpk, int cout, int cin)
{
    const int kcs = cin / 32;
    const int total = 3 * kcs * NFR * 64 * 8;
    for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += gridDim.x * blockDim.x) {
        const int e = idx & 7;
        const int lane = (idx >> 3) & 63;
        const int f = (idx >> 9) % NFR;
        const int kc = ((idx >> 9) / NFR) % kcs;
        const int ta = ((idx >> 9) / NFR) / kcs;
        const int n = 16 * f + (lane & 15);
        const int c = kc * 32 + (lane >> 4) * 8 + e;
        uint16_t v = 0;
        if (n < 27) {
            const int b = n / 9, d = (n % 9) / 3, o = n % 3;
            if (o < cout) v = w[((((int64_t)o * cin + c) * 3 + ta) * 3 + b) * 3 + d];
        }
        wpk[idx] = v;
    }
}
}  // namespace

hipError_t launch_pack_head(const void* w, void* wpk, int cout, int cin, hipStream_t s)
{
    const int total = (int)head_packed_elems(cin);
    hipLaunchKernelGGL(pack_head_kernel, dim3((total + 255) / 256), dim3(256), 0, s, (const uint16_t*)w,
                       (uint16_t*)wpk, cout, cin);
    return hipGetLastError();
}

hipError_t launch_conv_head(const ConvArgs& a, hipStream_t s)
{
    if (!head_conv_applies(a.cout, a.cin, a.kt, a.kh, a.kw, a.up_s)) return hipErrorInvalidValue;
    if (a.h_out != a.up_s * a.h_in || a.w_out != a.up_s * a.w_in || a.t_out < 1) return hipErrorInvalidValue;
    const int64_t ntiles = (int64_t)((a.h_in + TH - 1) / TH) * ((a.w_in + TW - 1) / TW);
    // a run of frames per workgroup: long runs read each input frame once; cut
    // them when there are too few tiles to fill the chip twice over
    int groups = (int)((2048 + ntiles - 1) / ntiles);
    if (groups > a.t_out) groups = a.t_out;
    if (groups < 1) groups = 1;
    const int fpw = (a.t_out + groups - 1) / groups;
    const int64_t total = ntiles * ((a.t_out + fpw - 1) / fpw);
    if (total > (int64_t)0x7fffffff - 8) return hipErrorInvalidValue;
    const int64_t grid = ((total + 7) / 8) * 8;
    const dim3 gd((unsigned)grid), bd(256);
    const int kc = a.cin / 32;
    if (a.up_s == 2) {
        if (kc == 1) hipLaunchKernelGGL((conv_head_kernel<2, 1>), gd, bd, 0, s, a, fpw);
        else if (kc == 2) hipLaunchKernelGGL((conv_head_kernel<2, 2>), gd, bd, 0, s, a, fpw);
        else if (kc == 3) hipLaunchKernelGGL((conv_head_kernel<2, 3>), gd, bd, 0, s, a, fpw);
        else return hipErrorInvalidValue;
    } else {
        if (kc == 1) hipLaunchKernelGGL((conv_head_kernel<1, 1>), gd, bd, 0, s, a, fpw);
        else if (kc == 2) hipLaunchKernelGGL((conv_head_kernel<1, 2>), gd, bd, 0, s, a, fpw);
        else if (kc == 3) hipLaunchKernelGGL((conv_head_kernel<1, 3>), gd, bd, 0, s, a, fpw);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cc3d
