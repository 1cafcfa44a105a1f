// Output-head conv on gfx950 MFMA: a 3x3x3 causal conv to at most three
// channels (RGB), on a nearest-2x upsampled input (UP = 2) or at the input's own
// size (UP = 1).
//
// With three output channels, the GEMM view of the other kernels (N = output
// channels) leaves 13 of 16 MFMA columns idle.  Here the spatial taps go into N
// instead: for every source pixel s of an input frame and every tap (a, b, d)
// and channel o,
//
//     P[s][(a, b, d, o)] = sum_c X[s][c] * W[o][c][a][b][d]
//
// is one GEMM with M = source pixels, K = Cin, N = 3 temporal x 9 spatial taps
// x 3 channels (27 per temporal tap, padded to 32).  An output pixel (y, x) of
// frame t then sums, for each tap, one entry of P: with UP = 2, spatial tap
// (b, d) of output phase (p, q) = (y & 1, x & 1) reads source (y/2 +
// floor((p+b-1)/2), x/2 + floor((q+d-1)/2)) -- nearest upsampling followed by
// zero padding of the upsampled image is exactly "zero outside the source
// image"; with UP = 1 it reads (y + b - 1, x + d - 1).  Temporal tap a reads
// input frame t + a of the causal window.  Every product of the conv's
// definition is formed once (in the MFMA) and every sum is taken in fp32, in a
// different order from the direct form; no weights are pre-summed.
//
// A workgroup owns a tile of 8 x 16 source pixels (16 x 32 output pixels, or
// 8 x 16 with UP = 1) and a run of consecutive output frames.  It walks the input frames of that run
// once: each frame's tile plus a one-pixel border (18 x 10 pixels, 12 M
// fragments) is loaded straight into MFMA operand registers (the next frame's
// while the current one is gathered), multiplied by the weights held in
// registers for the whole run, and the partial sums P go to LDS.  Each thread
// then gathers the taps of two horizontally adjacent output pixels (UP = 1: one
// pixel, threads 0..127) and adds them to a three-frame ring of fp32
// accumulators in registers; output frame t
// is complete, and stored (bf16, or the 8-bit code of the fp32 value), once
// input frame t + 2 has been added.
#include "cc3d_device.h"

namespace cc3d {
namespace {

constexpr int TH = 8, TW = 16;                  // source tile
constexpr int BH = TH + 2, BW = TW + 2;         // with the one-pixel border
constexpr int BPIX = BH * BW;                   // 180
constexpr int MFR = (BPIX + 15) / 16;           // 12 M fragments of 16 pixels
constexpr int MFW = MFR / 4;                    // 3 per wave
constexpr int NFR = 6;                          // 3 temporal taps x 32 columns
constexpr int PSTR = 100;                       // floats per pixel in the P table (96 used)

template <int UP, int KC>
__global__ __launch_bounds__(256, 2) void conv_head_kernel(ConvArgs a, int fpw)
{
    constexpr int NQ = UP;  // output pixels per thread (horizontal neighbours)
    __shared__ float ptab[MFR * 16 * PSTR];  // P[pixel of the bordered tile][n]

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
    // share their border rows and columns in L2 (measured 1-3% faster than
    // row-major order)
    constexpr int SR = 4;
    const int strip = tile / (SR * tiles_w), k = tile - strip * SR * tiles_w;
    const int sr = min(SR, tiles_h - strip * SR);
    const int i0 = (strip * SR + k % sr) * TH, j0 = (k / sr) * TW;
    const int t0 = tg * fpw;
    const int t1 = min(t0 + fpw, a.t_out);
    const int z0 = t0, z1 = t1 + 2;  // input frames of the causal window this run reads

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, k16 = lane & 15;

    // weights (MFMA row operand): row 16 f + k16, channels 32 kc + 8 g .. + 7
    bf16x8 wa[KC][NFR];
    const uint4* wp = (const uint4*)a.wpk;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int f = 0; f < NFR; ++f) wa[kc][f] = __builtin_bit_cast(bf16x8, wp[(kc * NFR + f) * 64 + lane]);

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
    bf16x8 xb[KC][MFW];
    auto load_frame = [&](int zi) {
        const uint16_t* fp = zframe(a.z, zi);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(fp, fp ? frame_bytes : 0u);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int mm = 0; mm < MFW; ++mm)
                xb[kc][mm] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(poff[mm] + (uint32_t)(kc * 64)), 0, 0));
    };

    // UP = 2: the two output pixels of this thread are row oy, columns 2 sj and
    // 2 sj + 1 of the 16 x 32 output tile (source row si, phase p = oy & 1).
    // UP = 1: threads 0..127 own output pixel (si, sj) of the 8 x 16 tile.
    const int oy = tid >> 4, sj = tid & 15;
    const int p = oy & 1, si = UP == 2 ? oy >> 1 : oy;
    const int Y = UP == 2 ? 2 * i0 + oy : i0 + oy, X = UP == 2 ? 2 * (j0 + sj) : j0 + sj;
    const bool row_ok = Y < a.h_out && (UP == 2 || tid < TH * TW);
    const int cout = a.cout;

    float ring[3][NQ][3];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int o = 0; o < 3; ++o) ring[s][q][o] = 0.f;

    auto store = [&](int t, const float (&v)[NQ][3]) {
        if (!row_ok) return;
        uint16_t* out = (uint16_t*)a.out;
        const uint16_t* res = (const uint16_t*)a.res;
        const int64_t base = (((int64_t)t * a.h_out + Y) * a.w_out + X) * cout;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (X + q >= a.w_out) continue;
#pragma unroll
            for (int o = 0; o < 3; ++o) {
                if (o >= cout) continue;
                float y = v[q][o];
                if (a.bias) y += a.bias[o];
                if (res) y += bf2f(res[base + q * cout + o]);
                if (a.out_u8)
                    ((uint8_t*)a.out)[base + q * cout + o] = rgb8_code(y);
                else
                    out[base + q * cout + o] = f2bf(y);
            }
        }
    };

    // One input frame zi at ring phase PH = (zi - z0) mod 3: output frame
    // t = zi - a takes temporal tap a; its accumulator is ring slot (t - z0) mod 3.
    auto frame = [&](const int zi, const int PH) {
        f32x4 acc[MFW][NFR];
#pragma unroll
        for (int mm = 0; mm < MFW; ++mm)
#pragma unroll
            for (int f = 0; f < NFR; ++f) acc[mm][f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int mm = 0; mm < MFW; ++mm)
#pragma unroll
                for (int f = 0; f < NFR; ++f)
                    acc[mm][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[kc][f], xb[kc][mm], acc[mm][f], 0, 0, 0);
        if (zi + 1 < z1) load_frame(zi + 1);
        __syncthreads();  // the previous frame's gather has finished reading P
        // acc[mm][f] = D[n][pixel]: lane (g, k16) holds n = 16 f + 4 g .. + 3 of pixel k16
#pragma unroll
        for (int mm = 0; mm < MFW; ++mm) {
            const int L = (wave * MFW + mm) * 16 + k16;
#pragma unroll
            for (int f = 0; f < NFR; ++f) *(f32x4*)&ptab[L * PSTR + 16 * f + 4 * g] = acc[mm][f];
        }
        __syncthreads();
        // gather.  UP = 2: tap (a, b, d) of output pixel (oy, 2 sj + q) reads
        // bordered-tile pixel (si + 1 + floor((p+b-1)/2), sj + 1 + floor((q+d-1)/2)):
        //   q = 0: d = 0 -> column sj, d = 1, 2 -> sj + 1;  q = 1: d = 0, 1 -> sj + 1, d = 2 -> sj + 2.
        // UP = 1: tap (a, b, d) of output pixel (si, sj) reads (si + b, sj + d).
#pragma unroll
        for (int ta = 0; ta < 3; ++ta) {
            const int t = zi - ta;
            if (t < t0 || t >= t1) continue;
            const int slot = ((PH - ta) % 3 + 3) % 3;
            if (UP == 2 || tid < TH * TW) {
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const int row = UP == 2 ? si + 1 + ((p + b - 1) >> 1) : si + b;
                    const float* pr = &ptab[(row * BW + sj) * PSTR + ta * 32 + b * 9];
#pragma unroll
                    for (int o = 0; o < 3; ++o) {
                        if (UP == 2) {
                            ring[slot][0][o] += pr[o] + pr[PSTR + 3 + o] + pr[PSTR + 6 + o];
                            ring[slot][NQ - 1][o] += pr[PSTR + o] + pr[PSTR + 3 + o] + pr[2 * PSTR + 6 + o];
                        } else {
                            ring[slot][0][o] += pr[o] + pr[PSTR + 3 + o] + pr[2 * PSTR + 6 + o];
                        }
                    }
                }
            }
            if (ta == 2) {  // output frame t has all its taps
                store(t, ring[slot]);
#pragma unroll
                for (int q = 0; q < NQ; ++q)
#pragma unroll
                    for (int o = 0; o < 3; ++o) ring[slot][q][o] = 0.f;
            }
        }
    };

    load_frame(z0);
    for (int zb = z0; zb < z1; zb += 3) {
        frame(zb, 0);
        if (zb + 1 < z1) frame(zb + 1, 1);
        if (zb + 2 < z1) frame(zb + 2, 2);
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
    return (size_t)(cin / 32) * NFR * 64 * 8;
}

namespace {
// Packed head weights: for each (32-channel chunk kc, N fragment f), 64 lanes of
// 8 channels: lane (g, k16) holds W[o][32 kc + 8 g + e][a][b][d] for row
// n = 16 f + k16 = 32 a + 3 (3 b + d) + o (zero for n mod 32 >= 27 or o >= cout).
__global__ void pack_head_kernel(const uint16_t* w, uint16_t* wpk, int cout, int cin)
{
    const int kcs = cin / 32;
    const int total = kcs * NFR * 64 * 8;
    for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += gridDim.x * blockDim.x) {
        const int e = idx & 7;
        const int lane = (idx >> 3) & 63;
        const int f = (idx >> 9) % NFR;
        const int kc = (idx >> 9) / NFR;
        const int n = 16 * f + (lane & 15);
        const int c = kc * 32 + (lane >> 4) * 8 + e;
        const int ta = n / 32, r = n % 32;
        uint16_t v = 0;
        if (r < 27) {
            const int tap = r / 3, o = r % 3;
            const int b = tap / 3, d = tap % 3;
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
