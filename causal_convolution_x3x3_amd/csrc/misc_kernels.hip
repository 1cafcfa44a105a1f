// Memory-bound kernels of the decode path: the fp32 direct conv (small fp32
// layers), the standalone channel RMSNorm + SiLU (+ residual) epilogue, the
// causal cache update, zero fill and the channels-first/last transposes.
#include "cc3d_device.h"

namespace cc3d {
namespace {

// ------------------------------------------------------------ fp32 conv ----
// One thread per output element (channel fastest, so neighbouring threads share
// their input reads); fp32 accumulation over taps, then channels.  Upsampled
// convs read source pixel floor(u / up_s) of upsampled pixel u; strided ones
// centre output (y, x) on input pixel (down_s*y, down_s*x) and output frame t on
// window frames t_stride*t + t_first + (0 .. kt-1).
__global__ __launch_bounds__(256) void conv_f32_kernel(ConvArgs a)
{
    const int64_t total = (int64_t)a.t_out * a.h_out * a.w_out * a.cout;
    const int ph = (a.kh - 1) / 2, pw = (a.kw - 1) / 2;
    const int hu = a.h_in * a.up_s, wu = a.w_in * a.up_s;  // the conv's input size
    const int kvol = a.kt * a.kh * a.kw;
    const float* w = (const float*)a.wpk;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int o = (int)(idx % a.cout);
        int64_t p = idx / a.cout;
        const int x = (int)(p % a.w_out);
        p /= a.w_out;
        const int y = (int)(p % a.h_out);
        const int t = (int)(p / a.h_out);
        float s = 0.f;
        for (int ta = 0; ta < a.kt; ++ta) {
            const float* fp = (const float*)zframe_bytes(a.z, a.t_stride * t + a.t_first + ta, 4);
            if (!fp) continue;
            for (int tb = 0; tb < a.kh; ++tb) {
                const int yu = a.down_s * y + tb - ph;
                if (yu < 0 || yu >= hu) continue;
                const int sy = yu / a.up_s;
                for (int td = 0; td < a.kw; ++td) {
                    const int xu = a.down_s * x + td - pw;
                    if (xu < 0 || xu >= wu) continue;
                    const int sx = xu / a.up_s;
                    const float* px = fp + ((int64_t)sy * a.w_in + sx) * a.cin;
                    const float* wp = w + (int64_t)o * a.cin * kvol + (ta * a.kh + tb) * a.kw + td;
                    for (int c = 0; c < a.cin; ++c) s = fmaf(px[c], wp[(int64_t)c * kvol], s);
                }
            }
        }
        if (a.bias) s += a.bias[o];
        if (a.res) s += ((const float*)a.res)[idx];
        ((float*)a.out)[idx] = s;
    }
}

// -------------------------------------------------------------- norm_act ---
// 32 lanes per pixel; lane u holds channel units u, u+32, ... of 4 channels.
constexpr int NORM_MAXU = 4;  // up to 512 channels

template <typename T>
struct Vec4;
template <>
struct Vec4<uint16_t> {
    static __device__ __forceinline__ void load(const void* p, int64_t e, float v[4]) {
        const uint2 r = *(const uint2*)((const uint16_t*)p + e);
        v[0] = bf2f((uint16_t)(r.x & 0xffffu));
        v[1] = bf2f((uint16_t)(r.x >> 16));
        v[2] = bf2f((uint16_t)(r.y & 0xffffu));
        v[3] = bf2f((uint16_t)(r.y >> 16));
    }
    static __device__ __forceinline__ void round(float v[4]) {
        for (int i = 0; i < 4; ++i) v[i] = bf2f(f2bf(v[i]));
    }
    static __device__ __forceinline__ void store(void* p, int64_t e, const float v[4]) {
        uint2 r;
        r.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        r.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *(uint2*)((uint16_t*)p + e) = r;
    }
};
template <>
struct Vec4<float> {
    static __device__ __forceinline__ void load(const void* p, int64_t e, float v[4]) {
        const float4 r = *(const float4*)((const float*)p + e);
        v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
    static __device__ __forceinline__ void round(float*) {}
    static __device__ __forceinline__ void store(void* p, int64_t e, const float v[4]) {
        *(float4*)((float*)p + e) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

template <typename T>
__global__ __launch_bounds__(256) void norm_act_kernel(NormArgs a)
{
    const int l32 = threadIdx.x & 31;
    const int64_t pix = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
    const bool live = pix < a.n_pix;
    const int nunits = a.c >> 2;
    float v[NORM_MAXU][4];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < NORM_MAXU; ++u) {
        const int unit = l32 + 32 * u;
        if (live && unit < nunits) {
            const int64_t e = pix * a.c + unit * 4;
            Vec4<T>::load(a.src, e, v[u]);
            if (a.res) {
                float r[4];
                Vec4<T>::load(a.res, e, r);
                for (int i = 0; i < 4; ++i) v[u][i] += r[i];
                Vec4<T>::round(v[u]);
            }
            for (int i = 0; i < 4; ++i) ss += v[u][i] * v[u][i];
        }
    }
    ss += __shfl_xor(ss, 1, 32);
    ss += __shfl_xor(ss, 2, 32);
    ss += __shfl_xor(ss, 4, 32);
    ss += __shfl_xor(ss, 8, 32);
    ss += __shfl_xor(ss, 16, 32);
    const float inv = 1.0f / sqrtf(ss / (float)a.c + a.eps);
#pragma unroll
    for (int u = 0; u < NORM_MAXU; ++u) {
        const int unit = l32 + 32 * u;
        if (live && unit < nunits) {
            const int64_t e = pix * a.c + unit * 4;
            const bool to_cache = a.cache && pix >= a.cache_pix0;
            const int64_t ce = (pix - a.cache_pix0) * a.c + unit * 4;
            if (a.out) Vec4<T>::store(a.out, e, v[u]);
            if (to_cache && !a.cache_act) Vec4<T>::store(a.cache, ce, v[u]);
            if (a.act_out) {
                float o[4];
                for (int i = 0; i < 4; ++i) {
                    const float z = a.gamma[unit * 4 + i] * v[u][i] * inv;
                    o[i] = z / (1.0f + expf(-z));
                }
                Vec4<T>::store(a.act_out, e, o);
                if (to_cache && a.cache_act) Vec4<T>::store(a.cache, ce, o);
            }
        }
    }
}

// ----------------------------------------------------- norm_act (bf16) ---
__device__ __forceinline__ void unpack8(const uint4& r, float v[8])
{
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint4 pack8(const float v[8])
{
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
}

// LPP lanes per pixel, each holding U 16-byte chunks (8 channels) of it: chunk
// l + LPP*u for lane l of the group, so C = 8 * LPP * U.  All loads of a thread
// are issued before its first store.
template <int LPP, int U>
__global__ __launch_bounds__(256) void norm_act_bf16_kernel(NormArgs a)
{
    const int l = threadIdx.x & (LPP - 1);
    const int64_t pix = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LPP;
    if (pix >= a.n_pix) return;  // whole LPP-lane groups leave together
    const uint4* src = (const uint4*)a.src + pix * (LPP * U);
    float v[U][8];
    uint4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = src[l + LPP * u];
    if (a.res) {
        const uint4* rs = (const uint4*)a.res + pix * (LPP * U);
        uint4 q[U];
#pragma unroll
        for (int u = 0; u < U; ++u) q[u] = rs[l + LPP * u];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float w[8];
            unpack8(r[u], v[u]);
            unpack8(q[u], w);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[u][i] += w[i];
            r[u] = pack8(v[u]);  // v is stored rounded; the act reads the rounded value
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        unpack8(r[u], v[u]);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += v[u][i] * v[u][i];
    }
#pragma unroll
    for (int o = 1; o < LPP; o <<= 1) ss += __shfl_xor(ss, o, LPP);
    const bool to_cache = a.cache && pix >= a.cache_pix0;
    uint4* cdst = (uint4*)a.cache + (pix - a.cache_pix0) * (LPP * U);
    if (a.out) {
        uint4* dst = (uint4*)a.out + pix * (LPP * U);
#pragma unroll
        for (int u = 0; u < U; ++u) dst[l + LPP * u] = r[u];
    }
    if (to_cache && !a.cache_act) {
#pragma unroll
        for (int u = 0; u < U; ++u) cdst[l + LPP * u] = r[u];
    }
    if (!a.act_out) return;
    const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / (float)a.c) + a.eps);
    uint4* dst = (uint4*)a.act_out + pix * (LPP * U);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c0 = 8 * (l + LPP * u);
        const float4 g0 = *(const float4*)(a.gamma + c0);
        const float4 g1 = *(const float4*)(a.gamma + c0 + 4);
        const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = silu(gm[i] * v[u][i] * inv);
        const uint4 h = pack8(o);
        dst[l + LPP * u] = h;
        if (to_cache && a.cache_act) cdst[l + LPP * u] = h;
    }
}

// (lanes per pixel, chunks per lane) for a bf16 norm over c channels, or false
// when c is not 8 * LPP * U with LPP in {4, 8, 16} and U <= 6.  The most lanes
// per pixel first: a load then covers 128 or 256 contiguous bytes of a pixel
// (measured 4% faster on 192 channels than 4 lanes x 6 chunks).
bool norm_bf16_shape(int c, int& lpp, int& u)
{
    if (c % 8 != 0) return false;
    const int chunks = c / 8;
    for (int cand : {16, 8, 4})
        if (chunks % cand == 0 && chunks / cand <= 6) {
            lpp = cand;
            u = chunks / cand;
            return true;
        }
    return false;
}

template <int LPP, int U>
hipError_t launch_norm_bf16(const NormArgs& a, hipStream_t s)
{
    const int64_t blocks = (a.n_pix * LPP + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((norm_act_bf16_kernel<LPP, U>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int LPP>
hipError_t launch_norm_bf16_u(const NormArgs& a, int u, hipStream_t s)
{
    switch (u) {
    case 1: return launch_norm_bf16<LPP, 1>(a, s);
    case 2: return launch_norm_bf16<LPP, 2>(a, s);
    case 3: return launch_norm_bf16<LPP, 3>(a, s);
    case 4: return launch_norm_bf16<LPP, 4>(a, s);
    case 5: return launch_norm_bf16<LPP, 5>(a, s);
    case 6: return launch_norm_bf16<LPP, 6>(a, s);
    default: return hipErrorInvalidValue;
    }
}

// ----------------------------------------------------------- cache update --
// dst[i] = Z[t_v + i] for i = 0 .. kt-2.  One thread moves element k of every
// frame, in ascending i, so dst may be the window's own cache (a frame batch
// that continues the cache it read): frame i is written after frame t_v + i > i
// was read, in the same thread.
template <typename V>
__global__ __launch_bounds__(256) void cache_update_kernel(ZWindow z, int t_v, void* dst, int eb)
{
    const int64_t n = z.frame_elems * eb / (int64_t)sizeof(V);
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n;
         k += (int64_t)gridDim.x * blockDim.x) {
        for (int i = 0; i < z.kt - 1; ++i) {
            const V* src = (const V*)zframe_bytes(z, t_v + i, eb);
            ((V*)dst)[i * n + k] = src ? src[k] : V{};
        }
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* d, int64_t n16, unsigned char* tail,
                                                        int ntail)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n16;
         k += (int64_t)gridDim.x * blockDim.x)
        d[k] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// -------------------------------------------------------------- transpose --
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* src, T* dst, int64_t rows,
                                                        int64_t cols)
{
    __shared__ T tile[32][33];
    const int64_t tiles_c = (cols + 31) / 32;
    const int64_t ntiles = tiles_c * ((rows + 31) / 32);
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    for (int64_t tb = blockIdx.x; tb < ntiles; tb += gridDim.x) {
        const int64_t r0 = (tb / tiles_c) * 32, c0 = (tb % tiles_c) * 32;
        __syncthreads();
        for (int j = ty; j < 32; j += 8) {
            const int64_t r = r0 + j, c = c0 + tx;
            if (r < rows && c < cols) tile[j][tx] = src[r * cols + c];
        }
        __syncthreads();
        for (int j = ty; j < 32; j += 8) {
            const int64_t c = c0 + j, r = r0 + tx;
            if (r < rows && c < cols) dst[c * rows + r] = tile[tx][j];
        }
    }
}

int grid_for(int64_t n, int per_block = 256, int cap = 1 << 20)
{
    int64_t b = (n + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

}  // namespace

hipError_t launch_conv_f32(const ConvArgs& a, hipStream_t s)
{
    const int64_t total = (int64_t)a.t_out * a.h_out * a.w_out * a.cout;
    hipLaunchKernelGGL(conv_f32_kernel, dim3(grid_for(total)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_norm_act(const NormArgs& a, int elem_bytes, hipStream_t s)
{
    if (a.c % 4 != 0 || a.c > 4 * 32 * NORM_MAXU) return hipErrorInvalidValue;
    const int64_t threads = a.n_pix * 32;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    int lpp = 0, u = 0;
    const bool aligned =
        (((uintptr_t)a.src | (uintptr_t)a.res | (uintptr_t)a.out | (uintptr_t)a.act_out | (uintptr_t)a.cache) & 15u) == 0;
    if (elem_bytes == 2 && aligned && norm_bf16_shape(a.c, lpp, u)) {
        if (lpp == 4) return launch_norm_bf16_u<4>(a, u, s);
        if (lpp == 8) return launch_norm_bf16_u<8>(a, u, s);
        return launch_norm_bf16_u<16>(a, u, s);
    }
    if (elem_bytes == 2)
        hipLaunchKernelGGL(norm_act_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(norm_act_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_cache_update(const ZWindow& z, int t_v, void* dst, int eb, hipStream_t s)
{
    if (z.kt <= 1) return hipSuccess;
    const int64_t bytes = z.frame_elems * eb;
    if (bytes % 16 == 0) {
        hipLaunchKernelGGL(cache_update_kernel<uint4>, dim3(grid_for(bytes / 16, 256, 8192)), dim3(256), 0, s, z,
                           t_v, dst, eb);
    } else {
        hipLaunchKernelGGL(cache_update_kernel<uint16_t>, dim3(grid_for(bytes / 2, 256, 8192)), dim3(256), 0, s, z,
                           t_v, dst, eb);
    }
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t s)
{
    const int64_t n16 = (int64_t)(bytes / 16);
    const int ntail = (int)(bytes % 16);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n16, 256, 8192)), dim3(256), 0, s, (uint4*)dst,
                       n16, (unsigned char*)dst + n16 * 16, ntail);
    return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int64_t rows, int64_t cols, int eb,
                            hipStream_t s)
{
    const int64_t ntiles = ((cols + 31) / 32) * ((rows + 31) / 32);
    const dim3 grid((unsigned)(ntiles < (1 << 20) ? (ntiles > 0 ? ntiles : 1) : (1 << 20)));
    if (eb == 2)
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)src,
                           (uint16_t*)dst, rows, cols);
    else if (eb == 4)
        hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)src,
                           (uint32_t*)dst, rows, cols);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace cc3d
