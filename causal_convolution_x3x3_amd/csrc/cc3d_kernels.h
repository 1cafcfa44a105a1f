// Internal interface between the host runtime (cc3d_api.cpp) and the gfx950
// kernels.  Not installed; the public C ABI is include/cc3d.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cc3d {

// The window a causal conv reads for one chunk: Z = history (kt-1 frames) ||
// V, where V is the chunk input grown in time (up_t = 2: V[u] = X[(u + t_shift)/2],
// i.e. first chunk V[0]=X[0], V[2j-1]=V[2j]=X[j] with t_shift = 1; later chunks,
// and the first one under the aligned rule, V[u]=X[u/2] with t_shift = 0).
// History is cache_in's frames, or on the video's first chunk zeros / copies of
// V[0].  Frames are at the input's own (pre-spatial-upsample) size.
struct ZWindow {
    const void* x;        // [T_in][H][W][C] chunk input
    const void* cache;    // [kt-1][H][W][C] cache_in frames (unused when first)
    int64_t frame_elems;  // H*W*C
    int kt;
    int up_t;
    int first;            // 1 on the video's first chunk
    int zero_hist;        // first-chunk history: 1 = zeros, 0 = copies of V[0]
    int t_shift;          // up_t = 2: V[u] = X[(u + t_shift) / 2]
};

struct ConvArgs {
    ZWindow z;
    const void* wpk;      // packed weights (layout depends on the kernel family)
    const float* bias;    // [cout] or null
    const void* res;      // [t_out][h_out][w_out][cout] or null
    void* out;            // result v = conv + bias (+ res), or null
    void* act_out;        // SiLU(RMSNorm(v)), or null (only when fused)
    const float* gamma;   // [cout]
    float eps;
    int cin, cout, kt, kh, kw;
    int h_in, w_in, up_s, h_out, w_out, t_out;
    int kchunks;          // bf16: ceil(cin / 32)
    int ntile, nblocks;   // bf16: output channels per workgroup, number of such blocks
    int family;           // bf16: kernel family (1 to 7) the weights were packed for
    int rot_taps;         // bf16 v2 and pointwise: rotate the temporal-tap order by the output frame
    int t_rot0;           // ... counted from this frame (the launch's first frame in its chunk)
    int out_u8;           // bf16 families 1 and 3: out holds 8-bit codes of the fp32 result
    // A later conv's cache written by this one (families 2, 5, 6, 7): output frames
    // t >= cache_t0 of the result (cache_act = 0) or of the act (1) are also
    // stored as frame t - cache_t0 of `cache`, or null.
    void* cache;
    int cache_t0;
    int cache_act;
    // Strided convs (bf16 families 1, 2, 6, 7 and fp32): output pixel (y, x) is centred on
    // input pixel (down_s*y, down_s*x); output frame t reads window frames
    // t_stride*t + t_first + (0 .. kt-1) of Z.  1, 1, 0 for every other conv.
    int down_s;
    int t_stride;
    int t_first;
};

// 8-bit output code of an fp32 result v: rint(clamp((v + 1) * 127.5, 0, 255)).
__device__ __forceinline__ uint8_t rgb8_code(float v)
{
    return (uint8_t)rintf(fminf(fmaxf((v + 1.0f) * 127.5f, 0.0f), 255.0f));
}

struct NormArgs {
    const void* src;      // [n_pix][c]
    const void* res;      // [n_pix][c] or null
    void* out;            // v = src (+ res) or null
    void* act_out;        // SiLU(RMSNorm(v)) or null
    const float* gamma;
    float eps;
    int64_t n_pix;
    int c;
    // A later conv's cache written by this pass: positions >= cache_pix0 of v
    // (cache_act = 0) or of the act (1) are also stored at position - cache_pix0
    // of `cache`, or null.
    void* cache;
    int64_t cache_pix0;
    int cache_act;
};

// bf16 implicit-GEMM conv on MFMA.  Returns hipErrorInvalidValue for a shape
// the kernel family does not take (the host checks bf16_conv_supported first).
bool bf16_conv_supported(int cout, int kh, int kw, int up_s);
void bf16_conv_tiling(int cout, int* ntile, int* nblocks);
hipError_t launch_conv_bf16(const ConvArgs& a, hipStream_t s);
// Repack [cout][cin][kt][kh][kw] bf16 weights into the MFMA operand blocks of
// the given kernel family.
size_t bf16_packed_elems(int cout, int cin, int kt, int kh, int kw, int family);
hipError_t launch_pack_bf16(const void* w, void* wpk, int cout, int cin, int kt, int kh, int kw,
                            int family, hipStream_t s);

// Register-blocked 3x3 spatial kernels (conv_bf16_v2.hip) for 96/128-channel
// output blocks; their weights are packed with the column tap outermost.
bool v2_conv_applies(int ntile, int kh, int kw, int up_s);
// Kernel family chosen for a bf16 conv: 3 = the output head (conv_head.hip)
// where it applies, 5 = the phase-decomposed upsample conv (conv_phase.hip)
// where it applies and `fold` != 0, 2 = v2 where it applies, 4 = the pointwise
// kernel (conv_pw.hip) for 1x1 spatial kernels whose epilogue is plain (no act,
// no 8-bit output: `plain` != 0), else 1.  CC3D_CONV_FAMILY=1 in the environment
// at plan creation keeps every conv on v1.  Strided convs are assigned by the
// host: 2 = v2's strided tile (96/128-channel blocks), 6 = the same with the
// temporal taps folded into one K step (8 input channels), 7 = v2's strided
// tile in 192-channel blocks (cout a multiple of 192), else 1.
int bf16_conv_family(int cout, int cin, int kt, int kh, int kw, int up_s, int plain, int fold);
hipError_t launch_conv_bf16_v2(const ConvArgs& a, hipStream_t s);

// Output head (conv_head.hip): 3x3x3 conv to at most 3 channels, of a nearest-2x
// upsampled input or at the input's own size, spatial taps in the GEMM's N
// dimension; weights packed per (32-channel chunk, N fragment) as 64 lanes x 8
// channels.
bool head_conv_applies(int cout, int cin, int kt, int kh, int kw, int up_s);
size_t head_packed_elems(int cin);
hipError_t launch_pack_head(const void* w, void* wpk, int cout, int cin, hipStream_t s);
hipError_t launch_conv_head(const ConvArgs& a, hipStream_t s);

// Pointwise kernel (conv_pw.hip): k_t x 1 x 1 convs, output channels in blocks
// of 192 (or 96); weights packed per (block, temporal tap, 64 channels).
bool pw_conv_applies(int cout, int kh, int kw, int up_s);
void pw_conv_tiling(int cout, int* ntile, int* nblocks);
size_t pw_packed_elems(int cout, int cin, int kt);
hipError_t launch_pack_pw(const void* w, void* wpk, int cout, int cin, int kt, hipStream_t s);
hipError_t launch_conv_pw(const ConvArgs& a, hipStream_t s);

// Phase-decomposed upsample conv (conv_phase.hip): 3x3 spatial, up_s = 2,
// 96-channel blocks; weights folded per output phase into hi/lo bf16 pairs.
bool phase_conv_applies(int ntile, int kh, int kw, int up_s);
size_t phase_packed_elems(int cout, int cin, int kt);
hipError_t launch_pack_phase(const void* w, void* wpk, int cout, int cin, int kt, hipStream_t s);
hipError_t launch_conv_phase(const ConvArgs& a, hipStream_t s);

// fp32 direct conv (weights used in PyTorch order, copied by the host).
hipError_t launch_conv_f32(const ConvArgs& a, hipStream_t s);

// v = src (+res); out = v; act_out = SiLU(RMSNorm(v)).  elem_bytes 2 (bf16) or 4.
hipError_t launch_norm_act(const NormArgs& a, int elem_bytes, hipStream_t s);

// cache_out[i] = Z[t_v + i], i < kt-1.
hipError_t launch_cache_update(const ZWindow& z, int t_v, void* dst, int elem_bytes,
                               hipStream_t s);

hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t s);

// dst[c][r] = src[r][c] for an rows x cols matrix of elem_bytes elements.
hipError_t launch_transpose(const void* src, void* dst, int64_t rows, int64_t cols,
                            int elem_bytes, hipStream_t s);

}  // namespace cc3d
