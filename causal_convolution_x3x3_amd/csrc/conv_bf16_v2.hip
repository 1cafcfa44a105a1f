// bf16 3x3x3 causal conv on gfx950 MFMA, register-blocked ("v2" family).
//
// Same GEMM view as conv_bf16.hip (M = output pixels, N = output channels,
// K = Cin x taps), built for throughput on the 3x3 spatial kernels that carry
// almost all of the decoder's FLOPs:
//
// * One workgroup of 8 waves per CU, two per SIMD so that one wave's LDS and
//   barrier waits are covered by the other's MFMAs.  Four waves along M each own
//   RH output rows x 16 columns (up_s = 1; RH = 9 for 96-channel blocks, 8 for
//   128) or RH source rows x 16 source columns at all four output phases
//   (up_s = 2; RH = 3 for 96-channel blocks, 2 for 128); the two waves along N
//   split the NTILE output channels.
// * K is walked in steps of (temporal tap a, 32 channels); each step in three
//   sub-steps, one per spatial column tap d.  A sub-step needs the step's input
//   tile (A, in LDS for the whole step) and the weights of the three taps (b, d),
//   b = 0..2 (B, 3 x NTILE x 32).  The next step's A goes from global memory
//   straight into an idle LDS buffer (buffer loads with the LDS flag) while the
//   current step runs; B goes through LDS the same way, two sub-steps ahead
//   where three buffers fit (else one); one barrier per sub-step.
// * The weights are the MFMA's row operand and the pixels its column operand,
//   so each lane's accumulators are four consecutive output channels of one
//   pixel: the epilogue moves 8-byte vectors.
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
// * Strided convs (DOWN = 2, the encoder side): the tile is RH output rows x 64
//   output columns, which read input rows 2y-1 .. 2y+1 and columns 2x-1 ..
//   2x+1.  The LDS tile keeps the even input columns first and the odd ones
//   after them, so a fragment's 16 output columns read 16 consecutive LDS
//   pixels at every column tap (even half at x + d/2 for d = 0, 2; odd half at x
//   for d = 1), and LDS row s serves output rows (s - b) / 2 for the row taps b
//   of the same parity.  Output frame t reads window frames
//   t_stride*t + t_first + (0 .. kt-1).
// * Folded temporal taps (TF, 8 input channels: the pixels padded to 8): the
//   K step's four 8-channel groups are the window frames t_stride*t + t_first
//   + g (g < kt; the fourth is zero), so the whole K is one step.  The LDS tile
//   is then planar, one plane of pixels per group, each plane a whole number of
//   64-slot rounds so that every wave's load reads one frame.
#include "cc3d_device.h"

namespace cc3d {
namespace {

// (tile, frame, channel block) of work item w; the channel block varies fastest.
__device__ __forceinline__ void decode_item(int w, int t_out, int nblocks, int& tile, int& t, int& nb)
{
    nb = w % nblocks;
    const int rest = w / nblocks;
    t = rest % t_out;
    tile = rest / t_out;
}

// Geometry of the two variants (per group of MW waves along M); RH = output
// rows per wave for up_s = 1, source rows per wave for up_s = 2.
template <int UP, int RH, int MW>
struct Geo;
template <int RH, int MW>
struct Geo<1, RH, MW> {  // tile: RH output rows x 16 MW columns; M-wave w: columns 16w..16w+15
    static constexpr int TS_H = RH, TS_W = 16 * MW;
    static constexpr int MF = RH;  // M fragments per wave: one per row
};
template <int RH, int MW>
struct Geo<2, RH, MW> {  // tile: 4 RH source rows x 16 source columns; M-wave w: source rows RH w .. RH w + RH-1
    static_assert(MW == 4, "the upsampling tile has four waves along M");
    static constexpr int TS_H = 4 * RH, TS_W = 16;
    static constexpr int MF = 4 * RH;  // RH rows x 4 phases
};

// MW = waves along M, WN = waves along N: the workgroup has MW*WN waves (8:
// two per SIMD); wave (wm, wn) computes M-wave wm's pixels for the NF/WN
// fragments of part wn.
//
// Staging: the input tile and the weights go from global memory straight into
// LDS (buffer loads with the LDS flag), so no registers or LDS stores are spent
// on them.  A thread's 16-byte slots are fixed (slot = tid + NT*it); the byte
// offset each slot reads inside a frame is computed once.  Every fragment read
// is a base register plus a constant (the chunk swizzle depends on the column
// only).  Weights are prefetched two sub-steps ahead (three LDS buffers; two,
// one sub-step ahead, where three do not fit), the input tile one K step ahead.
template <int UP, int NF, int WN, int RH, int DOWN, int TF, int MW>
__global__ __launch_bounds__(64 * MW * WN, 1) void conv3_v2_kernel(ConvArgs a)
{
    static_assert(DOWN == 1 || UP == 1, "a conv either upsamples or strides");
    static_assert(TF == 0 || DOWN == 2, "folded temporal taps: the strided tile only");
    static_assert(MW == 2 || MW == 4, "two or four waves along M");
    using G = Geo<UP, RH, MW>;
    constexpr int NT = 64 * MW * WN;    // threads
    constexpr int NFW = NF / WN;        // N fragments per wave
    // LDS tile: the input rows and columns the tile's outputs read
    constexpr int LH = DOWN == 2 ? 2 * G::TS_H + 1 : G::TS_H + 2;
    constexpr int LW = DOWN == 2 ? 2 * G::TS_W + 1 : G::TS_W + 2;
    constexpr int NE = (LW + 1) / 2;  // DOWN = 2: even input columns, stored first
    constexpr int LWP = (LW + 1) / 2 * 2;  // row pitch (pixels)
    constexpr int PL = (LH * LWP + 63) / 64 * 64;  // TF: pixels per plane, whole 64-slot rounds
    constexpr int ROWB = TF ? LWP * 16 : LWP * 64;  // bytes per LDS row (TF: of one plane)
    constexpr int NTILE = 16 * NF;
    constexpr int A_CH = TF ? 4 * PL : LH * LWP * 4;  // 16-byte slots of one LDS tile buffer
    constexpr int B_CH = 3 * NTILE * 4;     // 16-byte slots of one column tap's weights
    constexpr int A_IT = (A_CH + NT - 1) / NT;  // tile load rounds (16 bytes per lane)
    constexpr int A_PAD = A_IT * NT;            // tile buffer slots: whole rounds
    constexpr int B_BYTES = B_CH * 16;          // one column tap's weights
    constexpr int RB16 = B_CH / NT;             // weight load rounds of 16 bytes per lane ...
    constexpr int RB4 = (B_CH % NT) * 16 / (NT * 4);  // ... and of 4 bytes per lane for the rest
    static_assert(RB4 * NT * 4 == (B_CH % NT) * 16, "weight blocks split into whole load rounds");
    constexpr int RB = RB16 + RB4;              // weight load instructions per wave
    constexpr int MF = G::MF;
    constexpr int RED = WN * MW * MF * 16;      // epilogue reduction floats
    // weight buffers: 3 (prefetch distance 2) when they fit in LDS with the
    // double-buffered tile, else 2 (distance 1)
    // TF: one K step, so no tile is prefetched and the second tile buffer is unused
    constexpr int NA = TF ? 1 : 2;
    constexpr int NBB = (NA * A_PAD + 3 * B_CH) * 16 + RED * 4 <= 160 * 1024 ? 3 : 2;
    static_assert(NF % WN == 0, "N fragments split evenly over the N waves");

    // One LDS variable per buffer, and every load of the main loop issued
    // unconditionally (tile buffers padded to whole rounds; out-of-range slots
    // read zeros into the padding; the last steps reload instead of skipping):
    // the compiler's own waits then see exactly which loads are in flight, know
    // that the buffer being read is not one being filled, and add no waits.
    __shared__ uint4 lds_a0[A_PAD];
    __shared__ uint4 lds_a1[TF ? 1 : A_PAD];
    __shared__ uint4 lds_b0[B_CH];
    __shared__ uint4 lds_b1[B_CH];
    __shared__ uint4 lds_b2[NBB == 3 ? B_CH : 1];
    __shared__ float lds_red[RED];  // epilogue: per-pixel partial sums of squares

    // tiles cover the output frame (DOWN = 2) or the source frame (the output
    // frame too for UP = 1)
    const int tiles_w = ((DOWN == 2 ? a.w_out : a.w_in) + G::TS_W - 1) / G::TS_W;
    const int tiles_h = ((DOWN == 2 ? a.h_out : a.h_in) + G::TS_H - 1) / G::TS_H;
    const int total = tiles_w * tiles_h * a.t_out * a.nblocks;

  // One work item (tile, frame, channel block): main loop and epilogue.
  auto process = [&](const int w) {
    int tile, t, nb;
    decode_item(w, a.t_out, a.nblocks, tile, t, nb);
    const int i0 = (tile / tiles_w) * G::TS_H;  // tile origin (source frame for UP = 2, else output)
    const int j0 = (tile % tiles_w) * G::TS_W;
    // first window frame of output frame t
    const int tz0 = DOWN == 2 ? a.t_stride * t + a.t_first : t;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & (MW - 1), wn = wave / MW;
    const int g = lane >> 4, k16 = lane & 15;

    f32x4 acc[MF][NFW];
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
        for (int f = 0; f < NFW; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = TF ? 1 : a.kt * a.kchunks;
    const int nsub = nsteps * 3;
    const uint32_t frame_bytes = (uint32_t)(a.z.frame_elems * 2);
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc((const uint4*)a.wpk + (size_t)nb * nsub * B_CH, (uint32_t)(nsub * B_CH * 16));

    // Step-invariant load plan: byte offset inside a frame of the chunk slot
    // (tid + NT*it) holds (OOB: zero, i.e. outside the image or a padding column),
    // and the channel of its first element.
    uint32_t a_off[A_IT];
    int a_ch[A_IT];
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
        const int slot = tid + NT * it;
        a_off[it] = OOB;
        a_ch[it] = 0;
        if (TF && slot < A_CH) {
            // plane gg = window frame gg (the pixel's 8 channels)
            const int gg = slot / PL, pix = slot - gg * PL;
            const int r = pix / LWP, c = pix - r * LWP;
            a_ch[it] = gg;
            const int ci = c < NE ? 2 * c : 2 * (c - NE) + 1;
            const int gy = DOWN * i0 + r - 1, gx = DOWN * j0 + ci - 1;
            if (pix < LH * LWP && c < LW && gy >= 0 && gy < a.h_in && gx >= 0 && gx < a.w_in)
                a_off[it] = (uint32_t)((gy * a.w_in + gx) * a.cin * 2);
        } else if (!TF && slot < A_CH) {
            const int pix = slot >> 2;
            const int r = pix / LWP, c = pix - r * LWP;
            const int gg = (slot & 3) ^ swz(c);
            a_ch[it] = gg * 8;
            // input column of LDS column c (DOWN = 2: even columns, then odd)
            const int ci = DOWN == 2 ? (c < NE ? 2 * c : 2 * (c - NE) + 1) : c;
            const int gy = DOWN * i0 + r - 1, gx = DOWN * j0 + ci - 1;
            if (c < LW && gy >= 0 && gy < a.h_in && gx >= 0 && gx < a.w_in)
                a_off[it] = (uint32_t)(((gy * a.w_in + gx) * a.cin + gg * 8) * 2);
        }
    }

    // K steps take the temporal taps in an order rotated by the output frame:
    // loop step (ta, kc) reads tap (ta + rot) mod kt, rot = -(t_rot0 + t) mod kt
    // (the frame's place in its chunk, so a frame-batched run sums in the same
    // order as a whole-chunk one), so the
    // workgroups of frames t, t+1, t+2 -- which run at the same time -- read the
    // same input frame in the same step and share it in L2.
    const int rot = (!TF && a.rot_taps) ? (a.kt - (a.t_rot0 + tz0) % a.kt) % a.kt : 0;  // TF: one step
    auto phys_step = [&](int step) -> int {
        const int ta = step / a.kchunks, kc = step - ta * a.kchunks;
        const int tr = ta + rot < a.kt ? ta + rot : ta + rot - a.kt;
        return tr * a.kchunks + kc;
    };
    auto phys_sub = [&](int sub) -> int { return phys_step(sub / 3) * 3 + sub % 3; };
    auto issue_a = [&](int lstep, uint4* buf) {
        if (TF) {
            // one frame per load round and wave (the plane of its 64 slots)
#pragma unroll
            for (int it = 0; it < A_IT; ++it) {
                const int f = __builtin_amdgcn_readfirstlane(a_ch[it]);
                const uint16_t* fp = f < a.kt ? zframe(a.z, tz0 + f) : nullptr;
                load_to_lds(make_rsrc(fp, fp ? frame_bytes : 0u), a_off[it], buf + NT * it + wave * 64);
            }
            return;
        }
        const int step = phys_step(lstep);
        const int ta = step / a.kchunks, kc = step - ta * a.kchunks;
        const uint16_t* fp = zframe(a.z, tz0 + ta);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(fp, fp ? frame_bytes : 0u);
        const int ch0 = kc * 32;
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            const uint32_t off = (ch0 + a_ch[it] < a.cin) ? a_off[it] + (uint32_t)(ch0 * 2) : OOB;
            load_to_lds(r, off, buf + NT * it + wave * 64);
        }
    };
    // a column tap's weights, copied as they are packed: RB16 rounds of 16 bytes
    // per lane, then RB4 rounds of 4 bytes for what is left
    auto issue_b = [&](int lsub, uint4* buf) {
        const int sub = phys_sub(lsub);
#pragma unroll
        for (int it = 0; it < RB16; ++it)
            load_to_lds(wr, (uint32_t)((sub * B_CH + it * NT + tid) * 16), buf + it * NT + wave * 64);
#pragma unroll
        for (int it = 0; it < RB4; ++it)
            load_to_lds4(wr, (uint32_t)(sub * B_BYTES + RB16 * NT * 16 + (it * NT + tid) * 4),
                         (char*)buf + RB16 * NT * 16 + (it * NT + wave * 64) * 4);
    };
    // byte offset of this lane's 16-byte chunk at LDS column `col` of row 0
    auto col_off = [&](int col) -> int { return TF ? (g * PL + col) * 16 : col * 64 + ((g ^ swz(col)) << 4); };
    auto lds_frag = [&](const uint4* base, int byte_off) -> bf16x8 {
        return as_bf16x8(*(const uint4*)((const char*)base + byte_off));
    };
    int b_off[NFW];
#pragma unroll
    for (int f = 0; f < NFW; ++f) {
        const int nl = 16 * (wn * NFW + f) + k16;
        b_off[f] = nl * 64 + ((g ^ swz(nl)) << 4);
    }

    // The MFMAs of one sub-step (column tap d) from input buffer `aread` and the
    // B fragments bq[b][f] of taps (b, d).
    auto mma = [&](const int d, const uint4* aread, const bf16x8 (&bq)[3][NFW]) {
        if (DOWN == 2) {
            // LDS row s holds input row 2*i0 + s - 1; output row r reads rows 2r + b.
            const int base = col_off((d & 1) ? NE + 16 * wm + k16 : 16 * wm + k16 + (d >> 1));
#pragma unroll
            for (int s = 0; s < LH; ++s) {
                const bf16x8 av = lds_frag(aread, base + s * ROWB);
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const int r = (s - b) >> 1;
                    if (((s - b) & 1) == 0 && s >= b && r < G::TS_H) {
#pragma unroll
                        for (int f = 0; f < NFW; ++f)
                            acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[b][f], av, acc[r][f], 0, 0, 0);
                    }
                }
            }
        } else if (UP == 1) {
            // LDS row s holds source row i0 + s - 1; output row r reads rows r+b.
            const int base = col_off(16 * wm + k16 + d);
#pragma unroll
            for (int s = 0; s < G::TS_H + 2; ++s) {
                const bf16x8 av = lds_frag(aread, base + s * ROWB);
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const int r = s - b;
                    if (r >= 0 && r < G::TS_H) {
#pragma unroll
                        for (int f = 0; f < NFW; ++f)
                            acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[b][f], av, acc[r][f], 0, 0, 0);
                    }
                }
            }
        } else {
            // M fragment m = rr*4 + p*2 + q: source row R*wm + rr, phase (p, q).
            // Column offsets of this d: q=0 -> floor((d-1)/2), q=1 -> floor(d/2).
            // Each LDS row is read once and applied to every (rr, row tap) that
            // reads it: source row rr + oy with oy = floor((p+b-1)/2).
            constexpr int R = MF / 4;
            const int ox0 = (d - 1) >> 1, ox1 = d >> 1;
            const int base0 = col_off(k16 + ox0 + 1) + R * wm * ROWB;
            const int base1 = col_off(k16 + ox1 + 1) + R * wm * ROWB;
#pragma unroll
            for (int srow = 0; srow < R + 2; ++srow) {  // LDS row R*wm + srow: source row R*wm + srow - 1
                const bf16x8 a0 = lds_frag(aread, base0 + srow * ROWB);
                const bf16x8 a1 = (ox0 == ox1) ? a0 : lds_frag(aread, base1 + srow * ROWB);
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    const int oy = srow - 1 - rr;
                    if (oy < -1 || oy > 1) continue;
#pragma unroll
                    for (int p = 0; p < 2; ++p)
#pragma unroll
                        for (int b = 0; b < 3; ++b) {
                            if (((p + b - 1) >> 1) != oy) continue;
#pragma unroll
                            for (int f = 0; f < NFW; ++f) {
                                acc[rr * 4 + p * 2 + 0][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    bq[b][f], a0, acc[rr * 4 + p * 2 + 0][f], 0, 0, 0);
                                acc[rr * 4 + p * 2 + 1][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    bq[b][f], a1, acc[rr * 4 + p * 2 + 1][f], 0, 0, 0);
                            }
                        }
                }
            }
        }
    };

    // prologue: step 0's tile, the first NBB-1 sub-steps' weights
    issue_a(0, lds_a0);
    issue_b(0, lds_b0);
    if (NBB == 3) issue_b(nsub > 1 ? 1 : 0, lds_b1);
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    // One K step = three sub-steps (column taps d = 0, 1, 2), unrolled so the
    // tap and every LDS offset are compile-time constants; steps are taken in
    // pairs so that every buffer a sub-step reads or fills is a fixed LDS
    // variable.  Sub-step `sub` reads weight buffer sub % NBB and tile buffer
    // step % 2; it fills weight buffer (sub + NBB - 1) % NBB, last read in
    // sub-step sub - 1 (retired by its barrier), and at d = 0 the other tile
    // buffer, last read in the previous step.
    auto k_step = [&](int step, const uint4* aread, uint4* awrite, const int par) {
        const int next_a = step + 1 < nsteps ? step + 1 : 0;
        const int sub0 = 3 * step;
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            const int sub = sub0 + d;
            // NBB = 3: sub % 3 == d; NBB = 2: sub % 2 == (par + d) % 2 with par = step % 2.
            const int bcur = NBB == 3 ? d : ((par + d) & 1);
            const int bnext = NBB == 3 ? (d + 2) % 3 : (bcur ^ 1);
            const uint4* bread = bcur == 0 ? lds_b0 : (bcur == 1 ? lds_b1 : lds_b2);
            uint4* bwrite = bnext == 0 ? lds_b0 : (bnext == 1 ? lds_b1 : lds_b2);
            issue_b(sub + NBB - 1 < nsub ? sub + NBB - 1 : nsub - 1, bwrite);
            if (!TF && d == 0) issue_a(next_a, awrite);

            // B fragments of taps (b, d), b = 0..2, for this wave's channels
            bf16x8 bq[3][NFW];
#pragma unroll
            for (int b = 0; b < 3; ++b)
#pragma unroll
                for (int f = 0; f < NFW; ++f) bq[b][f] = lds_frag(bread, b_off[f] + b * NTILE * 64);
            mma(d, aread, bq);

            // Before the barrier: the weights of sub + 1 and, at d == 2, the
            // next tile must have landed.  Loads complete in issue order; the
            // loads issued after the ones needed may stay in flight.
            // (TF issues no tile in the loop: AT = 0)
            constexpr int AT = TF ? 0 : A_IT;
            if (NBB == 3) {
                // the weights of sub + 1 were issued in sub - 1, before
                // sub's weights (RB) and, at d <= 1, before the tile (AT)
                if (d == 2) wait_vmcnt<RB>();
                else wait_vmcnt<RB + AT>();
            } else {
                // the weights of sub + 1 were issued in this sub-step, before the tile
                if (d == 0) wait_vmcnt<AT>();
                else wait_vmcnt<0>();
            }
            // A bare barrier: the loads this barrier publishes were waited for
            // just above, every LDS read of this sub-step has been consumed by
            // its MFMA, and the loop issues no LDS stores, so __syncthreads'
            // release fence (which would drain the loads still in flight) is
            // not needed.
            __builtin_amdgcn_s_barrier();
        }
    };
    for (int step = 0; step < nsteps; step += 2) {
        k_step(step, lds_a0, lds_a1, 0);
        if (step + 1 < nsteps) k_step(step + 1, lds_a1, lds_a0, 1);
    }

    // ---------------------------------------------------------------- epilogue
    // The MFMAs above take the weights as the row operand, so acc[m][f] holds
    // D[channel][pixel]: lane (g, k16) has channels 16*F + 4g .. 16*F + 4g + 3
    // (F = wn*NFW + f) of pixel k16 of fragment m -- four consecutive channels,
    // moved with 8-byte loads and stores.
    //
    // v = acc + bias (+ res), rounded to bf16 and stored; the rounded value stays
    // in acc.  act = SiLU(RMSNorm(v)) from it: the sum of squares over a pixel's
    // channels is reduced in-lane, over the four lanes of that pixel (g), then
    // over the WN waves through LDS (the main loop's loads have all landed and its
    // reads retired, so lds_a0 is free).
    wait_vmcnt<0>();
    __syncthreads();
    const int n0 = nb * NTILE + wn * NFW * 16 + 4 * g;  // first channel of this lane in fragment f = 0
    uint16_t* out = (uint16_t*)a.out;
    uint16_t* act = (uint16_t*)a.act_out;
    const uint16_t* res = (const uint16_t*)a.res;
    // a later conv's cache: this frame's values also go to frame t - cache_t0 of
    // a.cache (the base is shifted so the same per-pixel offset applies)
    uint16_t* craw = nullptr;
    uint16_t* cact = nullptr;
    if (a.cache && t >= a.cache_t0) {
        uint16_t* cb = (uint16_t*)a.cache - (int64_t)a.cache_t0 * a.h_out * a.w_out * a.cout;
        if (a.cache_act) cact = cb;
        else craw = cb;
    }
    float* red = lds_red;  // [WN][MW][MF][16 pixels]
    const bool vec_ok = (a.cout & 3) == 0;  // 4-channel groups never straddle cout

    auto pixel_of = [&](int m, int& y, int& x) {
        if (UP == 1) {
            y = i0 + m;
            x = j0 + 16 * wm + k16;
        } else {
            const int rr = m >> 2, p = (m >> 1) & 1, q = m & 1;
            y = 2 * (i0 + (MF / 4) * wm + rr) + p;
            x = 2 * (j0 + k16) + q;
        }
    };
    auto pixel_base = [&](int m, bool& valid) -> int64_t {
        int y, x;
        pixel_of(m, y, x);
        valid = y < a.h_out && x < a.w_out;
        return (((int64_t)t * a.h_out + y) * a.w_out + x) * a.cout;
    };

    // The residual is loaded for the whole tile before anything is stored: the
    // compiler may not move a load of `res` past a store to `out` (they could
    // alias as far as it knows), so interleaved loads would each pay the full
    // memory latency.
    uint2 rv[MF][NFW];
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
        for (int f = 0; f < NFW; ++f) rv[m][f] = make_uint2(0u, 0u);
    if (res && vec_ok) {
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            bool valid;
            const int64_t pbase = pixel_base(m, valid);
#pragma unroll
            for (int f = 0; f < NFW; ++f) {
                const int n = n0 + 16 * f;
                if (valid && n < a.cout) rv[m][f] = *(const uint2*)(res + pbase + n);
            }
        }
    }

    // pass 1: v, stored; per-pixel partial sums of squares
#pragma clang loop unroll(full)
    for (int m = 0; m < MF; ++m) {
        bool valid;
        const int64_t pbase = pixel_base(m, valid);
        float ss = 0.f;
#pragma unroll
        for (int f = 0; f < NFW; ++f) {
            const int n = n0 + 16 * f;  // channels n .. n+3
            float v[4] = {acc[m][f][0], acc[m][f][1], acc[m][f][2], acc[m][f][3]};
            if (n < a.cout && vec_ok) {
                if (a.bias) {
                    const float4 bv = *(const float4*)(a.bias + n);
                    v[0] += bv.x; v[1] += bv.y; v[2] += bv.z; v[3] += bv.w;
                }
                if (res) {
                    v[0] += bf2f((uint16_t)(rv[m][f].x & 0xffffu));
                    v[1] += bf2f((uint16_t)(rv[m][f].x >> 16));
                    v[2] += bf2f((uint16_t)(rv[m][f].y & 0xffffu));
                    v[3] += bf2f((uint16_t)(rv[m][f].y >> 16));
                }
                const uint2 hb = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                v[0] = bf2f((uint16_t)(hb.x & 0xffffu));
                v[1] = bf2f((uint16_t)(hb.x >> 16));
                v[2] = bf2f((uint16_t)(hb.y & 0xffffu));
                v[3] = bf2f((uint16_t)(hb.y >> 16));
                if (out && valid) *(uint2*)(out + pbase + n) = hb;
                if (craw && valid) *(uint2*)(craw + pbase + n) = hb;
            } else if (n < a.cout) {  // cout not a multiple of 4: element by element
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (n + i >= a.cout) { v[i] = 0.f; continue; }
                    if (a.bias) v[i] += a.bias[n + i];
                    if (res && valid) v[i] += bf2f(res[pbase + n + i]);
                    const uint16_t hb = f2bf(v[i]);
                    v[i] = bf2f(hb);
                    if (out && valid) out[pbase + n + i] = hb;
                    if (craw && valid) craw[pbase + n + i] = hb;
                }
            } else {
                v[0] = v[1] = v[2] = v[3] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[m][f][i] = v[i];
                ss += v[i] * v[i];
            }
        }
        if (act) {
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            if (g == 0) red[((wn * MW + wm) * MF + m) * 16 + k16] = ss;
        }
    }
    if (!act) return;
    // act over 4-channel groups: act requires cout % 4 == 0 (checked on the host)
    float4 gm[NFW];
#pragma unroll
    for (int f = 0; f < NFW; ++f) {
        const int n = n0 + 16 * f;
        gm[f] = n < a.cout ? *(const float4*)(a.gamma + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float inv_c = 1.0f / (float)a.cout;
    __syncthreads();
    // pass 2: the act from the full channel sum
#pragma clang loop unroll(full)
    for (int m = 0; m < MF; ++m) {
        bool valid;
        const int64_t pbase = pixel_base(m, valid);
        float ss = 0.f;
#pragma unroll
        for (int h = 0; h < WN; ++h) ss += red[((h * MW + wm) * MF + m) * 16 + k16];
        const float inv = rms_scale(ss * inv_c, a.eps);
#pragma unroll
        for (int f = 0; f < NFW; ++f) {
            const int n = n0 + 16 * f;
            if (!valid || n >= a.cout) continue;
            const float z0 = silu(gm[f].x * acc[m][f][0] * inv), z1 = silu(gm[f].y * acc[m][f][1] * inv);
            const float z2 = silu(gm[f].z * acc[m][f][2] * inv), z3 = silu(gm[f].w * acc[m][f][3] * inv);
            const uint2 hv = make_uint2(pack_bf16x2(z0, z1), pack_bf16x2(z2, z3));
            *(uint2*)(act + pbase + n) = hv;
            if (cact) *(uint2*)(cact + pbase + n) = hv;
        }
    }
  };

    // Work items are dealt to the 8 XCDs in contiguous ranges (workgroups are
    // dealt to the XCDs round-robin), so neighbouring tiles and consecutive
    // frames run under the same L2.  With four or eight channel blocks (whose
    // weights together overflow one XCD's L2: 8 MB for a 384-channel layer),
    // block nb goes to the XCDs x with x % nblocks == nb instead, which split
    // that block's (tile, frame) items in contiguous ranges: each L2 then holds
    // one block's weights (measured on the 384-channel layers: 6-9% less fetch
    // from beyond L2, 63% less for the upsampling conv, time unchanged; with two
    // blocks the input re-read costs more than it saves).
    // (one call of process(): a second call site would keep the compiler from
    // inlining it)
    const int xcd = (int)(blockIdx.x & 7), slot = (int)(blockIdx.x >> 3);
    int w;
    bool live;
    if (a.nblocks == 4 || a.nblocks == 8) {
        const int share = 8 / a.nblocks;                  // XCDs per block
        const int items = total / a.nblocks;              // (tile, frame) items
        const int per = (items + share - 1) / share;
        const int j = (xcd / a.nblocks) * per + slot;
        live = slot < per && j < items;
        w = j * a.nblocks + xcd % a.nblocks;
    } else {
        w = xcd * ((total + 7) >> 3) + slot;
        live = w < total;
    }
    if (live) process(w);
}

template <int UP, int NF, int WN, int RH, int DOWN = 1, int TF = 0, int MW = 4>
hipError_t launch_v2(const ConvArgs& a, hipStream_t s)
{
    using G = Geo<UP, RH, MW>;
    const int th = DOWN == 2 ? a.h_out : a.h_in, tw = DOWN == 2 ? a.w_out : a.w_in;
    const int tiles = ((th + G::TS_H - 1) / G::TS_H) * ((tw + G::TS_W - 1) / G::TS_W);
    const int64_t total = (int64_t)tiles * a.t_out * a.nblocks;
    if (total <= 0 || total > (int64_t)0x7fffffff - 8) return hipErrorInvalidValue;
    const int64_t grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((conv3_v2_kernel<UP, NF, WN, RH, DOWN, TF, MW>), dim3((unsigned)grid), dim3(64 * MW * WN), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace

bool v2_conv_applies(int ntile, int kh, int kw, int up_s)
{
    return kh == 3 && kw == 3 && (up_s == 1 || up_s == 2) && (ntile == 96 || ntile == 128);
}

hipError_t launch_conv_bf16_v2(const ConvArgs& a, hipStream_t s)
{
    if (a.family == 7) {
        // spatial stride 2 in 192-channel blocks: 4 output rows x 32 columns per
        // tile (9 x 66 input pixels in LDS, double-buffered, beside two weight
        // buffers), two waves along M and four along N, each wave 4 rows x 16
        // columns x 48 channels: 18 fragment reads per 36 MFMAs per sub-step
        // against 14 per 18 for the 2-row tile
        if (a.ntile != 192 || a.kh != 3 || a.kw != 3 || a.down_s != 2 || a.up_s != 1 || a.t_stride < 1 ||
            a.t_stride > 2)
            return hipErrorInvalidValue;
        return launch_v2<1, 12, 4, 4, 2, 0, 2>(a, s);
    }
    if (!v2_conv_applies(a.ntile, a.kh, a.kw, a.up_s)) return hipErrorInvalidValue;
    if (a.down_s == 2) {
        // spatial stride 2: 2 output rows x 64 columns per tile (5 x 130 input
        // pixels in LDS, double-buffered, beside the weight buffers)
        if (a.up_s != 1 || a.t_stride < 1 || a.t_stride > 2) return hipErrorInvalidValue;
        if (a.family == 6) {  // 8 input channels, temporal taps folded into the K step
            if (a.cin != 8 || a.kt > 3) return hipErrorInvalidValue;
            // one K step: the tile is single-buffered, which leaves room for 4 rows
            return a.ntile == 96 ? launch_v2<1, 6, 2, 4, 2, 1>(a, s) : launch_v2<1, 8, 2, 4, 2, 1>(a, s);
        }
        return a.ntile == 96 ? launch_v2<1, 6, 2, 2, 2>(a, s) : launch_v2<1, 8, 2, 2, 2>(a, s);
    }
    if (a.family == 6) return hipErrorInvalidValue;
    if (a.t_stride != 1 || a.t_first != 0) return hipErrorInvalidValue;  // temporal stride: family 1
    // up_s = 1, 96-channel blocks: 9 output rows per wave (a 9 x 64 tile per
    // workgroup, weights three buffers deep in LDS).  Measured against 8 rows
    // (4-10% slower: fewer pixels per weight fetch, larger border share) and 10
    // rows (about 1% slower: the tile leaves room for two weight buffers only).
    // The 128-channel blocks keep 8 rows (more would not fit 256 VGPRs).
    //
    // A launch with fewer work items than CUs runs one item per busy CU, so its
    // time is one item's: for such small frames (the 90x160 residual block) the
    // tile is cut to 5 rows where that keeps the items within one wave of CUs,
    // which takes about 5/8 (5/9) of the time.  The sums per output pixel are
    // the same, in the same order, whichever tile computes it.
    if (a.up_s == 1) {
        const int64_t per_row_band = (int64_t)((a.w_in + 63) / 64) * a.t_out * a.nblocks;
        const int rh = a.ntile == 96 ? 9 : 8;
        const int64_t items = (a.h_in + rh - 1) / rh * per_row_band;
        const int64_t items5 = (a.h_in + 4) / 5 * per_row_band;
        const bool small = items < 256 && items5 <= 256;
        if (a.ntile == 96) return small ? launch_v2<1, 6, 2, 5>(a, s) : launch_v2<1, 6, 2, 9>(a, s);
        return small ? launch_v2<1, 8, 2, 5>(a, s) : launch_v2<1, 8, 2, 8>(a, s);
    }
    // up_s = 2, 96-channel blocks: three source rows per wave (measured 4%
    // faster than two rows; streaming the weights from L2 into registers instead
    // of LDS was slower in every variant: four waves then fetch the same weights).
    return a.ntile == 96 ? launch_v2<2, 6, 2, 3>(a, s) : launch_v2<2, 8, 2, 2>(a, s);
}

}  // namespace cc3d
