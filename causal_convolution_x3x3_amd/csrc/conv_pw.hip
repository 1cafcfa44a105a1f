// bf16 causal conv with a 1x1 spatial kernel (k_t x 1 x 1) on gfx950 MFMA:
// the pointwise ("pw") family.
//
// A conv whose spatial kernel is 1x1 mixes channels at each position and, for
// k_t > 1, across the frames of its causal window -- TemporalGrow's projection
// (1x1x1) and temporal conv (3x1x1) (LightX2V blog "SwiftVR Inference
// Optimization ...", section "TemporalGrow: Compute Before Spatial
// Upsampling").  Per output frame t this is a plain GEMM
//   Y[t][pos][n] = sum_{a, c} W[n][c][a] * Z[t + a][src(pos)][c]
// with M = the frame's positions, N = output channels, K = k_t x Cin, where Z is
// the causal window (history || input grown in time) and src() maps an output
// position to its source position (identity, or the nearest 2x upsample).
//
// * A work item is (a run of TP consecutive output positions of frame t, a block
//   of NTILE output channels).  8 waves: four along M (16*MW positions each)
//   and two along N; one workgroup per CU (two waves per SIMD) or, with a
//   smaller tile and ring, two (four waves per SIMD, so that one workgroup's
//   prologue and epilogue run beside the other's loop).  The weights are the MFMA's row operand, so
//   a lane's accumulators are four consecutive channels of one position and the
//   epilogue moves 8-byte vectors.
// * K is walked in steps of (temporal tap, 32 channels): one MFMA deep.  Both
//   operands go from global memory straight into LDS (buffer loads with the LDS
//   flag), NB - 1 steps ahead into a ring of NB buffer sets; one barrier per
//   step, which waits only for the next step's loads.  A step's MFMAs take well
//   under a microsecond, less than the loads' latency, so a deep ring (or a
//   second workgroup) is what keeps the pipe fed.  Every lane's 16-byte slot of the position tile has a
//   fixed source offset, so the nearest upsample (and any ragged tail past the
//   frame, read as zeros) costs nothing in the loop.
// * Temporal taps are taken in an order rotated by the output frame, and work
//   items run frame-major within a tile, so the workgroups of frames t, t+1, t+2
//   read the same input frame at the same time and share it in L2.  Items are
//   dealt to the 8 XCDs in contiguous ranges.
// * Epilogue: + bias, + residual, round to bf16 (nearest even) and store.  The
//   op's act and 8-bit output are not done here; the host picks this family only
//   for convs without them.
#include "cc3d_device.h"

namespace cc3d {
namespace {

template <int V>
struct IC {
    static constexpr int value = V;
};

constexpr int KC = 32;  // channels per K step

// NB = buffer sets in the ring (loads NB - 1 steps ahead, at most 5); OCC =
// workgroups per CU the LDS and registers are sized for.
template <int UP, int NF, int MW, int NB, int OCC>
__global__ __launch_bounds__(512, 2 * OCC) void conv_pw_kernel(ConvArgs a)
{
    constexpr int WN = 2, NT = 512;
    constexpr int NFW = NF / WN;          // N fragments per wave
    constexpr int NTILE = 16 * NF;
    constexpr int TP = 4 * 16 * MW;       // positions per work item
    constexpr int A_CH = TP * (KC / 8);   // 16-byte slots of one position-tile buffer
    constexpr int A_IT = A_CH / NT;
    constexpr int B_CH = NTILE * (KC / 8);  // 16-byte slots of one step's weights
    constexpr int B_BYTES = B_CH * 16;
    constexpr int RB16 = B_CH / NT;                   // weight rounds of 16 bytes per lane ...
    constexpr int RB4 = (B_CH % NT) * 16 / (NT * 4);  // ... then of 4 bytes for the rest
    static_assert(A_IT * NT == A_CH, "position tile in whole load rounds");
    static_assert(RB4 * NT * 4 == (B_CH % NT) * 16, "weight block in whole load rounds");
    static_assert(NF % WN == 0, "N fragments split evenly over the N waves");
    constexpr int LI = A_IT + RB16 + RB4;  // load instructions per step and lane
    static_assert((NB - 2) * LI < 64, "vmcnt range");
    static_assert(NB * (A_CH + B_CH) * 16 <= 160 * 1024 / OCC, "LDS budget");
    static_assert(NB >= 3 && NB <= 5, "three to five buffer sets");

    // one LDS variable per buffer (the compiler then sees which one a load fills)
    __shared__ uint4 lds_a0[A_CH], lds_a1[A_CH], lds_a2[A_CH], lds_a3[NB > 3 ? A_CH : 1], lds_a4[NB > 4 ? A_CH : 1];
    __shared__ uint4 lds_b0[B_CH], lds_b1[B_CH], lds_b2[B_CH], lds_b3[NB > 3 ? B_CH : 1], lds_b4[NB > 4 ? B_CH : 1];
    auto abuf = [&](auto J) -> uint4* {
        constexpr int j = decltype(J)::value;
        return j == 0 ? lds_a0 : j == 1 ? lds_a1 : j == 2 ? lds_a2 : j == 3 ? lds_a3 : lds_a4;
    };
    auto bbuf = [&](auto J) -> uint4* {
        constexpr int j = decltype(J)::value;
        return j == 0 ? lds_b0 : j == 1 ? lds_b1 : j == 2 ? lds_b2 : j == 3 ? lds_b3 : lds_b4;
    };

    const int hw_out = a.h_out * a.w_out;
    const int tiles = (hw_out + TP - 1) / TP;
    const int total = tiles * a.t_out * a.nblocks;
    const int per_xcd = (total + 7) >> 3;
    const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (w >= total) return;
    // (tile, frame, channel block) of item w; the channel block varies fastest,
    // then the frame
    const int nb = w % a.nblocks;
    const int t = (w / a.nblocks) % a.t_out;
    const int tile = w / a.nblocks / a.t_out;
    const int p0 = tile * TP;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;
    const int g = lane >> 4, k16 = lane & 15;

    const int kc_n = (a.cin + KC - 1) / KC;
    const int nsteps = a.kt * kc_n;
    const uint32_t frame_bytes = (uint32_t)(a.z.frame_elems * 2);
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc((const uint4*)a.wpk + (size_t)nb * nsteps * B_CH, (uint32_t)(nsteps * B_BYTES));

    // Step-invariant load plan: source byte offset inside a frame of the chunk
    // slot (tid + NT*it) holds (OOB past the frame's last position), and the
    // first channel of that chunk.
    uint32_t a_off[A_IT];
    int a_ch[A_IT];
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
        const int slot = tid + NT * it;
        const int pos = slot >> 2;
        const int chunk = (slot & 3) ^ swz(pos);
        const int op = p0 + pos;
        a_ch[it] = chunk * 8;
        a_off[it] = OOB;
        if (op < hw_out) {
            int src = op;
            if (UP == 2) {
                const int y = op / a.w_out, x = op - y * a.w_out;
                src = (y >> 1) * a.w_in + (x >> 1);
            }
            a_off[it] = (uint32_t)(((int64_t)src * a.cin + chunk * 8) * 2);
        }
    }

    // loop step (ta, kc) reads temporal tap (ta + rot) mod kt, rot = -(t_rot0 + t)
    // mod kt: the frame's place in its chunk
    const int rot = a.rot_taps ? (a.kt - (a.t_rot0 + t) % a.kt) % a.kt : 0;
    auto phys_step = [&](int step) -> int {
        const int ta = step / kc_n, kc = step - ta * kc_n;
        const int tr = ta + rot < a.kt ? ta + rot : ta + rot - a.kt;
        return tr * kc_n + kc;
    };
    auto issue = [&](int lstep, uint4* abuf, uint4* bbuf) {
        const int step = phys_step(lstep);
        const int ta = step / kc_n, kc = step - ta * kc_n;
        const uint16_t* fp = zframe(a.z, t + ta);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(fp, fp ? frame_bytes : 0u);
        const int ch0 = kc * KC;
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            const uint32_t off = (ch0 + a_ch[it] < a.cin) ? a_off[it] + (uint32_t)(ch0 * 2) : OOB;
            load_to_lds(r, off, abuf + NT * it + wave * 64);
        }
#pragma unroll
        for (int it = 0; it < RB16; ++it)
            load_to_lds(wr, (uint32_t)((step * B_CH + it * NT + tid) * 16), bbuf + it * NT + wave * 64);
#pragma unroll
        for (int it = 0; it < RB4; ++it)
            load_to_lds4(wr, (uint32_t)(step * B_BYTES + RB16 * NT * 16 + (it * NT + tid) * 4),
                         (char*)bbuf + RB16 * NT * 16 + (it * NT + wave * 64) * 4);
    };

    // byte offsets of this lane's fragments: the chunk of K group g in row
    // `row` is g ^ swz(row); rows of one lane differ by multiples of 16, so
    // swz is that of k16
    const int co = (g ^ swz(k16)) << 4;
    int a_frag[MW], b_frag[NFW];
#pragma unroll
    for (int m = 0; m < MW; ++m) a_frag[m] = (16 * MW * wm + 16 * m + k16) * 64 + co;
#pragma unroll
    for (int f = 0; f < NFW; ++f) b_frag[f] = (16 * (wn * NFW + f) + k16) * 64 + co;

    f32x4 acc[MW][NFW];
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int f = 0; f < NFW; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mma = [&](const uint4* ab, const uint4* bb) {
        bf16x8 bq[NFW];
#pragma unroll
        for (int f = 0; f < NFW; ++f) bq[f] = as_bf16x8(*(const uint4*)((const char*)bb + b_frag[f]));
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const bf16x8 av = as_bf16x8(*(const uint4*)((const char*)ab + a_frag[m]));
#pragma unroll
            for (int f = 0; f < NFW; ++f)
                acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[f], av, acc[m][f], 0, 0, 0);
        }
    };

    // Step s reads buffer set s % NB and fills set (s + NB - 1) % NB -- last read
    // in step s - 1, retired by its barrier -- with step s + NB - 1.  Steps past
    // the last reload the last one, so every load is unconditional and the
    // compiler's own waits stay exact; steps go in groups of NB so that every
    // buffer is a fixed LDS variable.
    auto clamp = [&](int s_) { return s_ < nsteps ? s_ : nsteps - 1; };
    issue(clamp(0), lds_a0, lds_b0);
    issue(clamp(1), lds_a1, lds_b1);
    if (NB > 3) issue(clamp(2), lds_a2, lds_b2);
    if (NB > 4) issue(clamp(3), lds_a3, lds_b3);
    wait_vmcnt<(NB - 2) * LI>();  // step 0 has landed
    __builtin_amdgcn_s_barrier();
    auto k_step = [&](int step, auto J) {
        constexpr int j = decltype(J)::value;
        issue(clamp(step + NB - 1), abuf(IC<(j + NB - 1) % NB>{}), bbuf(IC<(j + NB - 1) % NB>{}));
        mma(abuf(J), bbuf(J));
        // the next step's loads were issued NB - 1 steps ago; the NB - 2 later
        // steps' may stay in flight
        wait_vmcnt<(NB - 2) * LI>();
        // bare barrier: the loads it publishes were waited for just above and
        // the loop makes no LDS stores
        __builtin_amdgcn_s_barrier();
    };
    for (int step = 0; step < nsteps; step += NB) {
        k_step(step, IC<0>{});
        if (step + 1 < nsteps) k_step(step + 1, IC<1>{});
        if (step + 2 < nsteps) k_step(step + 2, IC<2>{});
        if constexpr (NB > 3) {
            if (step + 3 < nsteps) k_step(step + 3, IC<3>{});
        }
        if constexpr (NB > 4) {
            if (step + 4 < nsteps) k_step(step + 4, IC<4>{});
        }
    }

    // ---------------------------------------------------------------- epilogue
    // acc[m][f] holds D[channel][position]: lane (g, k16) has channels
    // n0 + 16 f .. + 3 of position p0 + 16 MW wm + 16 m + k16.
    const int n0 = nb * NTILE + wn * NFW * 16 + 4 * g;
    uint16_t* out = (uint16_t*)a.out;
    const uint16_t* res = (const uint16_t*)a.res;
#pragma unroll
    for (int m = 0; m < MW; ++m) {
        const int pos = p0 + 16 * MW * wm + 16 * m + k16;
        if (pos >= hw_out) continue;
        const int64_t pbase = ((int64_t)t * hw_out + pos) * a.cout;
        // this row's residual before its stores (a load of `res` may not move
        // past a store to `out`, which could alias it as far as the compiler knows)
        uint2 rv[NFW];
#pragma unroll
        for (int f = 0; f < NFW; ++f) {
            const int n = n0 + 16 * f;
            rv[f] = make_uint2(0u, 0u);
            if (res && n < a.cout) rv[f] = *(const uint2*)(res + pbase + n);
        }
#pragma unroll
        for (int f = 0; f < NFW; ++f) {
            const int n = n0 + 16 * f;
            if (n >= a.cout) continue;
            float v[4] = {acc[m][f][0], acc[m][f][1], acc[m][f][2], acc[m][f][3]};
            if (a.bias) {
                const float4 bv = *(const float4*)(a.bias + n);
                v[0] += bv.x; v[1] += bv.y; v[2] += bv.z; v[3] += bv.w;
            }
            if (res) {
                v[0] += bf2f((uint16_t)(rv[f].x & 0xffffu));
                v[1] += bf2f((uint16_t)(rv[f].x >> 16));
                v[2] += bf2f((uint16_t)(rv[f].y & 0xffffu));
                v[3] += bf2f((uint16_t)(rv[f].y >> 16));
            }
            *(uint2*)(out + pbase + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
    }
}

template <int UP, int NF, int MW = 4, int NB = 5, int OCC = 1>
hipError_t launch_pw(const ConvArgs& a, hipStream_t s)
{
    constexpr int TP = 4 * 16 * MW;
    const int64_t hw = (int64_t)a.h_out * a.w_out;
    const int64_t total = (hw + TP - 1) / TP * a.t_out * a.nblocks;
    if (total <= 0 || total > (int64_t)0x7fffffff - 8) return hipErrorInvalidValue;
    const int64_t grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((conv_pw_kernel<UP, NF, MW, NB, OCC>), dim3((unsigned)grid), dim3(512), 0, s, a);
    return hipGetLastError();
}

// Packed layout per (channel block, temporal tap, 32-channel chunk): NTILE rows
// of 32 channels, the 16-byte chunks of row nl swizzled by swz(nl) as in LDS;
// zero past cout and cin.
__global__ void pack_pw_kernel(const uint16_t* w, uint16_t* wpk, int cout, int cin, int kt, int ntile,
                               int nblocks, int kc_n)
{
    const int64_t total = (int64_t)nblocks * kt * kc_n * ntile * KC;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int e = (int)(idx % KC);
        int64_t row = idx / KC;
        const int nl = (int)(row % ntile);
        row /= ntile;
        const int kc = (int)(row % kc_n);
        row /= kc_n;
        const int ta = (int)(row % kt);
        const int nb = (int)(row / kt);
        const int chunk = (e >> 3) ^ swz(nl);
        const int c = kc * KC + chunk * 8 + (e & 7);
        const int n = nb * ntile + nl;
        uint16_t v = 0;
        if (n < cout && c < cin) v = w[((int64_t)n * cin + c) * kt + ta];
        wpk[idx] = v;
    }
}

}  // namespace

bool pw_conv_applies(int cout, int kh, int kw, int up_s)
{
    return kh == 1 && kw == 1 && (up_s == 1 || up_s == 2) && cout % 96 == 0;
}

void pw_conv_tiling(int cout, int* ntile, int* nblocks)
{
    const int nt = cout % 192 == 0 ? 192 : 96;
    *ntile = nt;
    *nblocks = cout / nt;
}

size_t pw_packed_elems(int cout, int cin, int kt)
{
    int nt, nb;
    pw_conv_tiling(cout, &nt, &nb);
    return (size_t)nb * kt * ((cin + KC - 1) / KC) * nt * KC;
}

hipError_t launch_pack_pw(const void* w, void* wpk, int cout, int cin, int kt, hipStream_t s)
{
    int nt, nb;
    pw_conv_tiling(cout, &nt, &nb);
    const size_t total = pw_packed_elems(cout, cin, kt);
    int blocks = (int)((total + 255) / 256);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(pack_pw_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t*)w, (uint16_t*)wpk, cout,
                       cin, kt, nt, nb, (cin + KC - 1) / KC);
    return hipGetLastError();
}

hipError_t launch_conv_pw(const ConvArgs& a, hipStream_t s)
{
    if (!pw_conv_applies(a.cout, a.kh, a.kw, a.up_s) || a.act_out || a.out_u8 || !a.out) return hipErrorInvalidValue;
    // 192-channel blocks: 384 positions per item (each wave 96 positions x 96
    // channels: 12 fragment reads per 36 MFMAs), a ring of three buffer sets
    // (108 KB), one workgroup per CU -- measured 6-10% faster on TemporalGrow's
    // convs than 128 positions with two workgroups per CU (8 reads per 12 MFMAs,
    // bound by LDS bandwidth), and than 256 positions with five sets or 384 with four
    if (a.ntile == 192) return a.up_s == 1 ? launch_pw<1, 12, 6, 3, 1>(a, s) : launch_pw<2, 12, 6, 3, 1>(a, s);
    if (a.ntile == 96) return a.up_s == 1 ? launch_pw<1, 6>(a, s) : launch_pw<2, 6>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace cc3d
