// Phase-decomposed 3x3x3 upsample conv on gfx950 MFMA (the "phase" family).
//
// A 3x3 spatial conv of a nearest-2x upsampled input gives, at output phase
// (p, q) = (y & 1, x & 1), a conv of the *source* image over the 2 x 2 source
// offsets (oy, ox), oy in {p-1, p}, ox in {q-1, q}: spatial tap (b, d) reads
// source offset (floor((p+b-1)/2), floor((q+d-1)/2)) (the same map the
// upsampling kernels use), so the taps that share an offset can be summed
// first.  Per phase the nine taps fold into four weights, made of 1, 2, 2 and 4
// taps.  Summed in fp32 and split into hi = bf16(W') and lo = bf16(W' - hi), a
// folded weight is W' to about 2^-17 relative (a single tap: lo = 0, not
// computed), so seven bf16 operands per phase and temporal tap replace nine:
// 7/9 of the MFMA work of the definition, with results equal to it up to fp32
// rounding.
//
// The same holds in time: where two or three temporal taps of an output frame
// read the same input frame of the causal window (the nearest 2x temporal
// growth repeats every frame; a first chunk's history repeats its first frame),
// which the window's frame pointers show, their weights are summed too.  Weights
// are packed for every tap alone, for the pairs (0, 1) and (1, 2) and for the
// three together; each work item groups its taps by frame and walks the groups.
// A group of several taps makes every lo non-zero, so the grouping variant
// (launched for convs that double the frame count, where nearly every output
// frame has one pair and one single tap) applies all eight operands per group:
// 16 of the 27 operand applications per output pixel instead of 21.
//
// The kernel is the register-blocked conv of conv_bf16_v2.hip at the source
// resolution (RH source rows x 64 source columns per workgroup, 8 waves: 4
// along M, 2 along N), with one output phase per work item: work items are
// (tile, frame, channel block, phase), phase fastest, so the four phases of a
// tile read the same input tile from L2.  A K step (temporal group, 32 channels)
// has two sub-steps, one per source column offset, each applying up to four
// operands (hi and lo of the two row offsets) to the LDS rows of the tile.
// Staging (buffer loads straight into LDS, one step ahead for the tile, one
// sub-step ahead for the weights), the temporal-tap rotation, the XCD work
// order and the epilogue (bias, residual, bf16 store, fused RMSNorm + SiLU when
// one block holds every channel) are those of the v2 kernel.
#include "cc3d_device.h"

namespace cc3d {
namespace {

template <int V>
struct IC {
    static constexpr int value = V;
};

// Taps of a 3-tap axis that phase `ph` (0 or 1) folds into source offset
// o = ph - 1 + k (k = 0, 1): 1 or 2 of them.
__host__ __device__ constexpr int fold_count(int ph, int k) { return (k == ph) ? 1 : 2; }

constexpr int NOP = 4;  // operands per sub-step: hi and lo of the two row offsets

// Temporal weight sets: taps 0 .. kt-1 alone, then (kt = 2) the pair (0, 1), or
// (kt = 3) the pairs (0, 1) and (1, 2) and the triple (0, 1, 2).
__host__ __device__ constexpr int num_wsets(int kt) { return kt == 3 ? 6 : (kt == 2 ? 3 : 1); }
__host__ __device__ inline void wset_taps(int kt, int w, int& a0, int& a1)
{
    a0 = a1 = w;
    if (w < kt) return;
    if (kt == 2) { a0 = 0; a1 = 1; return; }
    if (w == 3) { a0 = 0; a1 = 1; }
    else if (w == 4) { a0 = 1; a1 = 2; }
    else { a0 = 0; a1 = 2; }
}

// TF: group temporal taps that read the same frame (launched for convs that grow
// time; without it every tap is its own group and no branch is compiled in).
template <int NF, int RH, bool TF>
__global__ __launch_bounds__(512, 1) void conv_phase_kernel(ConvArgs a)
{
    constexpr int WN = 2, NT = 512;
    constexpr int NFW = NF / WN;
    constexpr int TS_H = RH, TS_W = 64, MF = RH;
    constexpr int LH = TS_H + 2, LW = TS_W + 2;
    constexpr int LWP = (LW + 1) / 2 * 2;
    constexpr int ROWB = LWP * 64;
    constexpr int NTILE = 16 * NF;
    constexpr int A_CH = LH * LWP * 4;
    constexpr int A_IT = (A_CH + NT - 1) / NT;
    constexpr int A_PAD = A_IT * NT;
    constexpr int B_CH = NOP * NTILE * 4;   // 16-byte slots of one sub-step's weights
    constexpr int RB = B_CH / NT;           // weight load rounds (16 bytes per lane)
    static_assert(RB * NT == B_CH, "weight block in whole load rounds");
    constexpr int RED = WN * 4 * MF * 16;
    static_assert((2 * A_PAD + 2 * B_CH) * 16 + RED * 4 <= 160 * 1024, "LDS budget");

    __shared__ uint4 lds_a0[A_PAD];
    __shared__ uint4 lds_a1[A_PAD];
    __shared__ uint4 lds_b0[B_CH];
    __shared__ uint4 lds_b1[B_CH];
    __shared__ float lds_red[RED];

    const int tiles_w = (a.w_in + TS_W - 1) / TS_W;
    const int tiles_h = (a.h_in + TS_H - 1) / TS_H;
    const int nbp = a.nblocks * 4;  // (channel block, phase) pairs, phase fastest
    const int total = tiles_w * tiles_h * a.t_out * nbp;
    const int per_xcd = (total + 7) >> 3;
    const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (w >= total) return;
    const int nbq = w % nbp;
    const int t = (w / nbp) % a.t_out;
    const int tile = w / nbp / a.t_out;
    const int ph = nbq & 3, cb = nbq >> 2;
    const int i0 = (tile / tiles_w) * TS_H, j0 = (tile % tiles_w) * TS_W;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;
    const int g = lane >> 4, k16 = lane & 15;

    // Temporal taps grouped by the input frame they read: group i starts at tap
    // g_taps >> 4i & 15 and uses weight set g_sets >> 4i & 15 (bit fields rather
    // than a table, which the compiler would place in per-lane memory).  Window
    // frames are told apart by the source frame they hold, not by address: frame
    // zi >= kt-1 holds input frame (zi - (kt-1) + t_shift) / 2; with replicated
    // history the history frames hold the first input frame (first chunk) or the
    // previous window's last grown pair, one source frame that no frame of this
    // window holds.  A frame-batched run, which reads from the cache what a
    // whole-chunk run reads from the input, then groups alike.  Under zero history
    // whether the two history frames hold one source frame depends on how the
    // video began, which a replayed graph could not follow: no grouping there.
    int ng = a.kt;
    uint32_t g_taps = 0x210u, g_sets = 0x210u;
    if (TF && !a.z.zero_hist) {
        const int hist = a.kt - 1;
        auto fid = [&](int zi) -> int {
            if (zi >= hist) return (zi - hist + a.z.t_shift) >> 1;
            return a.z.first ? 0 : -1;
        };
        const int z0 = fid(t), z1 = fid(t + 1), z2 = fid(t + 2);
        if (a.kt == 3) {
            if (z0 == z1 && z1 == z2) { ng = 1; g_taps = 0x0u; g_sets = 0x5u; }
            else if (z0 == z1) { ng = 2; g_taps = 0x20u; g_sets = 0x23u; }
            else if (z1 == z2) { ng = 2; g_taps = 0x10u; g_sets = 0x40u; }
        } else if (a.kt == 2 && z0 == z1) {
            ng = 1; g_taps = 0x0u; g_sets = 0x2u;
        }
    }
    const int nws = num_wsets(a.kt);
    const int nsteps = ng * a.kchunks;
    const int nsub = nsteps * 2;
    const int wsub = nws * a.kchunks * 2;  // packed sub-steps of one (channel block, phase)
    const uint32_t frame_bytes = (uint32_t)(a.z.frame_elems * 2);
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc((const uint4*)a.wpk + (size_t)(cb * 4 + ph) * wsub * B_CH, (uint32_t)(wsub * B_CH * 16));

    uint32_t a_off[A_IT];
    int a_ch[A_IT];
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
        const int slot = tid + NT * it;
        a_off[it] = OOB;
        a_ch[it] = 0;
        if (slot < A_CH) {
            const int pix = slot >> 2;
            const int r = pix / LWP, c = pix - r * LWP;
            const int gg = (slot & 3) ^ swz(c);
            a_ch[it] = gg * 8;
            const int gy = i0 + r - 1, gx = j0 + c - 1;
            if (c < LW && gy >= 0 && gy < a.h_in && gx >= 0 && gx < a.w_in)
                a_off[it] = (uint32_t)(((gy * a.w_in + gx) * a.cin + gg * 8) * 2);
        }
    }
    // groups taken in an order rotated by the output frame's place in the chunk
    // (from the group holding tap -(t_rot0 + t) mod kt), so the workgroups of
    // neighbouring frames read the same input frame at about the same time
    const int rot = a.rot_taps ? (a.kt - (a.t_rot0 + t) % a.kt) % a.kt : 0;
    // the group holding tap rot: the number of later groups' first taps <= rot
    const int g_first = !TF ? rot
                            : (ng > 1 && rot >= (int)(g_taps >> 4 & 15u)) + (ng > 2 && rot >= (int)(g_taps >> 8 & 15u));
    auto group_of = [&](int step, int& tap, int& set, int& kc) {
        const int gl = step / a.kchunks;
        kc = step - gl * a.kchunks;
        int gi = g_first + gl;
        if (gi >= ng) gi -= ng;
        tap = (int)(g_taps >> (4 * gi) & 15u);
        set = (int)(g_sets >> (4 * gi) & 15u);
    };
    auto issue_a = [&](int lstep, uint4* buf) {
        int ta, set, kc;
        group_of(lstep, ta, set, kc);
        const uint16_t* fp = zframe(a.z, t + ta);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(fp, fp ? frame_bytes : 0u);
        const int ch0 = kc * 32;
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            const uint32_t off = (ch0 + a_ch[it] < a.cin) ? a_off[it] + (uint32_t)(ch0 * 2) : OOB;
            load_to_lds(r, off, buf + NT * it + wave * 64);
        }
    };
    auto issue_b = [&](int lsub, uint4* buf) {
        int ta, set, kc;
        group_of(lsub >> 1, ta, set, kc);
        const int sub = (set * a.kchunks + kc) * 2 + (lsub & 1);
#pragma unroll
        for (int it = 0; it < RB; ++it)
            load_to_lds(wr, (uint32_t)((sub * B_CH + it * NT + tid) * 16), buf + it * NT + wave * 64);
    };
    auto col_off = [&](int col) -> int { return col * 64 + ((g ^ swz(col)) << 4); };
    auto lds_frag = [&](const uint4* base, int byte_off) -> bf16x8 {
        return as_bf16x8(*(const uint4*)((const char*)base + byte_off));
    };
    int b_off[NFW];
#pragma unroll
    for (int f = 0; f < NFW; ++f) {
        const int nl = 16 * (wn * NFW + f) + k16;
        b_off[f] = nl * 64 + ((g ^ swz(nl)) << 4);
    }

    f32x4 acc[MF][NFW];
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
        for (int f = 0; f < NFW; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Main loop for output phase (P, Q).  Sub-step s takes source column offset
    // ox = Q - 1 + s (LDS column shift Q + s); LDS row srow serves output row
    // r = srow - bs for the row shifts bs = P and P + 1 (row offset bs - 1).
    // Operands of a sub-step: 0 = hi and 1 = lo of row shift P, 2 = hi and 3 =
    // lo of row shift P + 1; a lo is zero, and skipped, where one tap (one
    // temporal tap and one spatial tap) folds.
    auto main_loop = [&](auto PC, auto QC) {
        constexpr int P = decltype(PC)::value, Q = decltype(QC)::value;
        // with temporal grouping every lo is applied: a group of several taps
        // makes each lo non-zero, and a test per step would split the MFMA chain
        auto mma = [&](auto SC, const uint4* aread, const bf16x8 (&bq)[NOP][NFW]) {
            constexpr int S = decltype(SC)::value;
            const int base = col_off(16 * wm + k16 + Q + S);
#pragma unroll
            for (int srow = 0; srow < TS_H + 2; ++srow) {
                const bf16x8 av = lds_frag(aread, base + srow * ROWB);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int r = srow - (P + k);
                    if (r < 0 || r >= TS_H) continue;
#pragma unroll
                    for (int f = 0; f < NFW; ++f)
                        acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[2 * k][f], av, acc[r][f], 0, 0, 0);
                    if (TF || fold_count(P, k) * fold_count(Q, S) > 1) {
#pragma unroll
                        for (int f = 0; f < NFW; ++f)
                            acc[r][f] =
                                __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[2 * k + 1][f], av, acc[r][f], 0, 0, 0);
                    }
                }
            }
        };
        // one K step: two sub-steps; sub-step s reads weight buffer s and, in
        // s = 0, fills the other one with the next sub-step's weights; the tile
        // for the next step goes into the idle tile buffer at s = 0
        auto k_step = [&](int step, const uint4* aread, uint4* awrite) {
            const int next_a = step + 1 < nsteps ? step + 1 : 0;
            const int sub0 = 2 * step;
            bf16x8 bq[NOP][NFW];
            // s = 0: weights in b0; prefetch the weights of s = 1 into b1, then the next tile
            issue_b(sub0 + 1, lds_b1);
            issue_a(next_a, awrite);
#pragma unroll
            for (int o = 0; o < NOP; ++o)
#pragma unroll
                for (int f = 0; f < NFW; ++f) bq[o][f] = lds_frag(lds_b0, b_off[f] + o * NTILE * 64);
            mma(IC<0>{}, aread, bq);
            wait_vmcnt<A_IT>();  // the weights of s = 1 (issued before the tile) have landed
            __builtin_amdgcn_s_barrier();
            // s = 1: weights in b1; prefetch the next step's s = 0 weights into b0
            issue_b(sub0 + 2 < nsub ? sub0 + 2 : nsub - 1, lds_b0);
#pragma unroll
            for (int o = 0; o < NOP; ++o)
#pragma unroll
                for (int f = 0; f < NFW; ++f) bq[o][f] = lds_frag(lds_b1, b_off[f] + o * NTILE * 64);
            mma(IC<1>{}, aread, bq);
            wait_vmcnt<0>();  // the next step's tile and first weights have landed
            __builtin_amdgcn_s_barrier();
        };
        issue_a(0, lds_a0);
        issue_b(0, lds_b0);
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        for (int step = 0; step < nsteps; step += 2) {
            k_step(step, lds_a0, lds_a1);
            if (step + 1 < nsteps) k_step(step + 1, lds_a1, lds_a0);
        }
    };
    switch (ph) {
    case 0: main_loop(IC<0>{}, IC<0>{}); break;
    case 1: main_loop(IC<0>{}, IC<1>{}); break;
    case 2: main_loop(IC<1>{}, IC<0>{}); break;
    default: main_loop(IC<1>{}, IC<1>{}); break;
    }

    // ---------------------------------------------------------------- epilogue
    // As in the v2 kernel: acc[m][f] holds D[channel][pixel], lane (g, k16) has
    // channels n0 + 16 f .. + 3 of source pixel (i0 + m, j0 + 16 wm + k16), i.e.
    // output pixel (2 (i0 + m) + P, 2 (j0 + 16 wm + k16) + Q).
    wait_vmcnt<0>();
    __syncthreads();
    const int P = ph >> 1, Q = ph & 1;
    const int n0 = cb * NTILE + wn * NFW * 16 + 4 * g;
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
    float* red = lds_red;
    const bool vec_ok = (a.cout & 3) == 0;
    auto pixel_base = [&](int m, bool& valid) -> int64_t {
        const int y = 2 * (i0 + m) + P, x = 2 * (j0 + 16 * wm + k16) + Q;
        valid = y < a.h_out && x < a.w_out;
        return (((int64_t)t * a.h_out + y) * a.w_out + x) * a.cout;
    };
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
#pragma clang loop unroll(full)
    for (int m = 0; m < MF; ++m) {
        bool valid;
        const int64_t pbase = pixel_base(m, valid);
        float ss = 0.f;
#pragma unroll
        for (int f = 0; f < NFW; ++f) {
            const int n = n0 + 16 * f;
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
            } else if (n < a.cout) {
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
            if (g == 0) red[((wn * 4 + wm) * MF + m) * 16 + k16] = ss;
        }
    }
    if (!act) return;
    float4 gm[NFW];
#pragma unroll
    for (int f = 0; f < NFW; ++f) {
        const int n = n0 + 16 * f;
        gm[f] = n < a.cout ? *(const float4*)(a.gamma + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float inv_c = 1.0f / (float)a.cout;
    __syncthreads();
#pragma clang loop unroll(full)
    for (int m = 0; m < MF; ++m) {
        bool valid;
        const int64_t pbase = pixel_base(m, valid);
        float ss = 0.f;
#pragma unroll
        for (int h = 0; h < WN; ++h) ss += red[((h * 4 + wm) * MF + m) * 16 + k16];
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
}

// Packed weights per (channel block, phase, temporal weight set, 32-channel
// chunk, sub-step s, operand o): NTILE rows of 32 channels, 16-byte chunks
// swizzled as in LDS.  Phase ph = 2 P + Q; sub-step s is source column offset
// Q - 1 + s; operand o = 2 k + l is the folded weight of row offset P - 1 + k,
// hi (l = 0) or lo (l = 1): W' = the fp32 sum over the set's temporal taps and
// the spatial taps (b, d) that read that offset, hi = bf16(W'), lo = bf16(W' - hi).
__global__ void pack_phase_kernel(const uint16_t* w, uint16_t* wpk, int cout, int cin, int kt, int ntile,
                                  int nblocks, int kchunks)
{
    const int nws = num_wsets(kt);
    const int64_t total = (int64_t)nblocks * 4 * nws * kchunks * 2 * NOP * ntile * 32;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int e = (int)(idx & 31);
        int64_t row = idx >> 5;
        const int nl = (int)(row % ntile);
        row /= ntile;
        const int o = (int)(row % NOP);
        row /= NOP;
        const int s = (int)(row % 2);
        row /= 2;
        const int kc = (int)(row % kchunks);
        row /= kchunks;
        const int ws = (int)(row % nws);
        row /= nws;
        const int ph = (int)(row % 4);
        const int cb = (int)(row / 4);
        const int P = ph >> 1, Q = ph & 1;
        const int k = o >> 1, lo = o & 1;
        const int oy = P - 1 + k, ox = Q - 1 + s;
        const int c = kc * 32 + (((e >> 3) ^ swz(nl)) << 3) + (e & 7);
        const int n = cb * ntile + nl;
        uint16_t v = 0;
        if (n < cout && c < cin) {
            int a0, a1;
            wset_taps(kt, ws, a0, a1);
            float sum = 0.f;
            for (int ta = a0; ta <= a1; ++ta)
                for (int b = 0; b < 3; ++b) {
                    if (((P + b - 1) >> 1) != oy) continue;
                    for (int d = 0; d < 3; ++d) {
                        if (((Q + d - 1) >> 1) != ox) continue;
                        sum += bf2f(w[((((int64_t)n * cin + c) * kt + ta) * 3 + b) * 3 + d]);
                    }
                }
            const uint16_t hi = f2bf(sum);
            v = lo ? f2bf(sum - bf2f(hi)) : hi;
        }
        wpk[idx] = v;
    }
}

}  // namespace

bool phase_conv_applies(int ntile, int kh, int kw, int up_s)
{
    return kh == 3 && kw == 3 && up_s == 2 && ntile == 96;
}

size_t phase_packed_elems(int cout, int cin, int kt)
{
    int nt, nb;
    bf16_conv_tiling(cout, &nt, &nb);
    return (size_t)nb * 4 * num_wsets(kt) * ((cin + 31) / 32) * 2 * NOP * nt * 32;
}

hipError_t launch_pack_phase(const void* w, void* wpk, int cout, int cin, int kt, hipStream_t s)
{
    int nt, nb;
    bf16_conv_tiling(cout, &nt, &nb);
    const size_t total = phase_packed_elems(cout, cin, kt);
    int blocks = (int)((total + 255) / 256);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(pack_phase_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t*)w, (uint16_t*)wpk, cout,
                       cin, kt, nt, nb, (cin + 31) / 32);
    return hipGetLastError();
}

hipError_t launch_conv_phase(const ConvArgs& a, hipStream_t s)
{
    if (!phase_conv_applies(a.ntile, a.kh, a.kw, a.up_s) || a.kt > 3 || a.out_u8) return hipErrorInvalidValue;
    if (a.h_out != 2 * a.h_in || a.w_out != 2 * a.w_in) return hipErrorInvalidValue;
    // temporal taps can read one frame only where the conv doubles time (or on a
    // first chunk's history, which the ungrouped variant simply reads again)
    const bool tf = a.z.up_t == 2;
    constexpr int RH = 9;
    const int64_t tiles = (int64_t)((a.h_in + RH - 1) / RH) * ((a.w_in + 63) / 64);
    const int64_t total = tiles * a.t_out * a.nblocks * 4;
    if (total <= 0 || total > (int64_t)0x7fffffff - 8) return hipErrorInvalidValue;
    const int64_t grid = ((total + 7) / 8) * 8;
    if (tf) hipLaunchKernelGGL((conv_phase_kernel<6, RH, true>), dim3((unsigned)grid), dim3(512), 0, s, a);
    else hipLaunchKernelGGL((conv_phase_kernel<6, RH, false>), dim3((unsigned)grid), dim3(512), 0, s, a);
    return hipGetLastError();
}

}  // namespace cc3d
