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
// three frames (output frame t reads frames t, t+1, t+2; frame t+3 is requested
// into frame t's slot as soon as t's products are formed).  The weights sit in
// LDS (copied once per workgroup).  P goes to one of two LDS buffers: in the
// step of output frame t a thread forms the products of frame t+1 with its
// gather of frame t's taps interleaved, writes frame t+1's P to the other
// buffer and stores frame t; one barrier per frame.  Measured on the 1440p
// head (8 x 16 tiles over 26 window frames): the kernel takes within a few
// percent of a copy of the same loads alone, which run at about 5 TB/s for this
// tile shape (2-D tiles with a border read below the contiguous-stream rate).
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

constexpr int RING = 3;                         // window frames held in registers

// Epilogue variants: the common RGB heads (three channels, no residual) store
// without a runtime branch, which lets the compiler interleave one frame's
// gather with the next frame's MFMAs; anything else takes the general path.
enum { EPI_GENERAL = 0, EPI_RGB_BF16 = 1, EPI_RGB_U8 = 2 };

template <int UP, int KC, int EPI>
__global__ __launch_bounds__(256, 2) void conv_head_kernel(ConvArgs a, int fpw)
{
    __shared__ float ptab[2 * PBUF];
    __shared__ uint4 wlds[3 * KC * NFR * 64];

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

    // weights (MFMA row operand) to LDS: for temporal tap ta, chunk kc and
    // fragment f, lane (g, k16) reads row 16 f + k16, channels 32 kc + 8 g .. + 7
    {
        const uint4* wp = (const uint4*)a.wpk;
        for (int i = tid; i < 3 * KC * NFR * 64; i += 256) wlds[i] = wp[i];
    }

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
    bf16x8 xb[RING][KC][MFW];
    // Every call issues its loads: a frame past the run's window reads through an
    // empty descriptor (zeros, no memory traffic).  With no load behind a branch
    // in the main loop, the compiler's wait counts follow the ring exactly
    // (a conditional load makes it wait for every load still in flight).
    auto load_frame = [&](const int zi, const int slot) {
        const uint16_t* fp = zi < z1 ? zframe(a.z, zi) : nullptr;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(fp, fp ? frame_bytes : 0u);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int mm = 0; mm < MFW; ++mm)
                xb[slot][kc][mm] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(poff[mm] + (uint32_t)(kc * 64)), 0, 0));
    };

    f32x4 acc[MFW][NFR];  // P of one output frame
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
    // UP = 1: thread tid owns output pixel (si, sj) of the 8 x 16 tile, tid & 127
    // (threads 128..255 repeat the gather of threads 0..127 and store nothing:
    // the gather then has no branch around it).
    constexpr int NQ = UP;
    const int oy = (UP == 2 ? tid : tid & 127) >> 4, sj = tid & 15;
    const int p = oy & 1, si = UP == 2 ? oy >> 1 : oy;
    const int Y = UP == 2 ? 2 * i0 + oy : i0 + oy, X = UP == 2 ? 2 * (j0 + sj) : j0 + sj;
    const bool mine = Y < a.h_out && X < a.w_out && (UP == 2 || tid < TH * TW);

    // products_gather: the products of the frame whose first window frame is in
    // ring slot s0 (with `prod`), tap ta = i interleaved with row tap b = i of
    // the gather from P buffer pb (with `gath`), so the gather's LDS reads and
    // adds issue while the MFMAs run.
    // Gather: UP = 2: tap (b, d) of output pixel (oy, 2 sj + q) reads
    // bordered-tile pixel (si + 1 + floor((p+b-1)/2), sj + 1 + floor((q+d-1)/2)):
    //   q = 0: d = 0 -> column sj, d = 1, 2 -> sj + 1;  q = 1: d = 0, 1 -> sj + 1, d = 2 -> sj + 2.
    // UP = 1: tap (b, d) of output pixel (si, sj) reads (si + b, sj + d).
    auto products_gather = [&](const int s0, const float* pb, float (&v)[NQ][3], const bool prod,
                               const bool gath) {
#pragma unroll
        for (int mm = 0; mm < MFW; ++mm)
#pragma unroll
            for (int f = 0; f < NFR; ++f) acc[mm][f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int o = 0; o < 3; ++o) v[q][o] = bias[o];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (prod) {
                bf16x8 wa[KC][NFR];  // temporal tap i's weights, read together
#pragma unroll
                for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                    for (int f = 0; f < NFR; ++f)
                        wa[kc][f] = __builtin_bit_cast(bf16x8, wlds[((i * KC + kc) * NFR + f) * 64 + lane]);
#pragma unroll
                for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                    for (int f = 0; f < NFR; ++f)
#pragma unroll
                        for (int mm = 0; mm < MFW; ++mm)
                            acc[mm][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                wa[kc][f], xb[(s0 + i) % RING][kc][mm], acc[mm][f], 0, 0, 0);
            }
            if (!gath) continue;
            const int b = i;
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
    };

    auto store = [&](const int t, float (&v)[NQ][3]) {
        if (!mine) return;
        const int64_t base = (((int64_t)t * a.h_out + Y) * a.w_out + X) * cout;
        if (EPI == EPI_RGB_BF16 && UP == 2) {
            // 6 values of two neighbouring pixels from an even element (X and
            // w_out are even): three 4-byte stores
            uint32_t* o32 = (uint32_t*)((uint16_t*)a.out + base);
            o32[0] = pack_bf16x2(v[0][0], v[0][1]);
            o32[1] = pack_bf16x2(v[0][2], v[NQ - 1][0]);
            o32[2] = pack_bf16x2(v[NQ - 1][1], v[NQ - 1][2]);
            return;
        }
        if (EPI == EPI_RGB_U8 && UP == 2) {
            uint16_t* o8 = (uint16_t*)((uint8_t*)a.out + base);
            o8[0] = (uint16_t)(rgb8_code(v[0][0]) | (rgb8_code(v[0][1]) << 8));
            o8[1] = (uint16_t)(rgb8_code(v[0][2]) | (rgb8_code(v[NQ - 1][0]) << 8));
            o8[2] = (uint16_t)(rgb8_code(v[NQ - 1][1]) | (rgb8_code(v[NQ - 1][2]) << 8));
            return;
        }
        if (EPI == EPI_RGB_BF16) {
#pragma unroll
            for (int o = 0; o < 3; ++o) ((uint16_t*)a.out)[base + o] = f2bf(v[0][o]);
            return;
        }
        if (EPI == EPI_RGB_U8) {
#pragma unroll
            for (int o = 0; o < 3; ++o) ((uint8_t*)a.out)[base + o] = rgb8_code(v[0][o]);
            return;
        }
        const uint16_t* res = (const uint16_t*)a.res;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (X + q >= a.w_out) continue;
#pragma unroll
            for (int o = 0; o < 3; ++o) {
                if (o >= cout) continue;
                float y = v[q][o];
                if (res) y += bf2f(res[base + q * cout + o]);
                if (a.out_u8)
                    ((uint8_t*)a.out)[base + q * cout + o] = rgb8_code(y);
                else
                    ((uint16_t*)a.out)[base + q * cout + o] = f2bf(y);
            }
        }
    };

    // Output frame t (ring slot of its first window frame: PH = (t - t0) mod RING).
    // On entry P of frame t is being written to buffer (t - t0) & 1.  Every step
    // but the run's last forms the products of frame t+1 (the MFMAs run while the
    // same wave gathers frame t's taps from LDS), requests window frame t+1+RING
    // into the slot frame t+1 leaves, writes frame t+1's P to the other buffer,
    // and stores frame t.
    auto step = [&](const int t, const int PH) {
        __syncthreads();  // P of frame t is complete; every gather of frame t-1 is done
        float v[NQ][3];
        products_gather((PH + 1) % RING, ptab + ((t - t0) & 1) * PBUF, v, true, true);
        load_frame(t + 1 + RING, (PH + 1) % RING);
        write_p(ptab + ((t + 1 - t0) & 1) * PBUF);
        store(t, v);
    };

#pragma unroll
    for (int r = 0; r < RING; ++r) load_frame(t0 + r, r);
    __syncthreads();  // the weights are in LDS
    {
        float unused[NQ][3];
        products_gather(0, ptab, unused, true, false);  // the run's first frame
    }
    load_frame(t0 + RING, 0);
    write_p(ptab);
    int tb = t0;
    for (; tb + RING < t1; tb += RING) {  // whole groups of steps that have a next frame
#pragma unroll
        for (int r = 0; r < RING; ++r) step(tb + r, r);
    }
#pragma unroll
    for (int r = 0; r < RING - 1; ++r)
        if (tb + r < t1 - 1) step(tb + r, r);
    __syncthreads();
    float v[NQ][3];
    products_gather(0, ptab + ((t1 - 1 - t0) & 1) * PBUF, v, false, true);  // the run's last frame
    store(t1 - 1, v);
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
    const int epi = (a.cout == 3 && !a.res) ? (a.out_u8 ? EPI_RGB_U8 : EPI_RGB_BF16) : EPI_GENERAL;
#define CC3D_HEAD_LAUNCH(UPV, KCV, EPIV) \
    hipLaunchKernelGGL((conv_head_kernel<UPV, KCV, EPIV>), gd, bd, 0, s, a, fpw)
#define CC3D_HEAD_EPI(UPV, KCV)                                        \
    do {                                                               \
        if (epi == EPI_RGB_BF16) CC3D_HEAD_LAUNCH(UPV, KCV, EPI_RGB_BF16); \
        else if (epi == EPI_RGB_U8) CC3D_HEAD_LAUNCH(UPV, KCV, EPI_RGB_U8); \
        else CC3D_HEAD_LAUNCH(UPV, KCV, EPI_GENERAL);                  \
    } while (0)
    if (a.up_s == 2) {
        if (kc == 1) CC3D_HEAD_EPI(2, 1);
        else if (kc == 2) CC3D_HEAD_EPI(2, 2);
        else if (kc == 3) CC3D_HEAD_EPI(2, 3);
        else return hipErrorInvalidValue;
    } else {
        if (kc == 1) CC3D_HEAD_EPI(1, 1);
        else if (kc == 2) CC3D_HEAD_EPI(1, 2);
        else if (kc == 3) CC3D_HEAD_EPI(1, 3);
        else return hipErrorInvalidValue;
    }
#undef CC3D_HEAD_EPI
#undef CC3D_HEAD_LAUNCH
    return hipGetLastError();
}

}  // namespace cc3d
