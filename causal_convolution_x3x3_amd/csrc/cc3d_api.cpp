// Host runtime of the C ABI in include/cc3d.h: argument validation (always
// before any device work), plan construction (weight repack, intermediate
// slots, cache arena layout), and the per-chunk launch sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/cc3d.h"
#include "cc3d_kernels.h"

namespace {

thread_local char g_err[1024] = "";

cc3d_status fail(cc3d_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

void clear_err() { g_err[0] = 0; }

constexpr uint32_t kPlanMagic = 0xCC3D0A11u;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Frame count of a slot for one chunk: T = (mul * t_chunk + (first ? add_first :
// add_rest)) / div, a chunk length being valid only where that is a whole number
// (strided convs halve the count).
struct FrameCount {
    int64_t mul = 0, add_first = 0, add_rest = 0, div = 1;
    bool operator==(const FrameCount& o) const {
        return mul == o.mul && add_first == o.add_first && add_rest == o.add_rest && div == o.div;
    }
    int64_t num(int64_t t, bool first) const { return mul * t + (first ? add_first : add_rest); }
    bool whole(int64_t t, bool first) const { return num(t, first) % div == 0; }
    int64_t eval(int64_t t, bool first) const { return num(t, first) / div; }
    // an upper bound for chunks of up to t frames (buffer sizing)
    int64_t bound(int64_t t) const {
        return (std::max(num(t, true), num(t, false)) + div - 1) / div;
    }
    // nearest 2x in time on non-first frames (every frame with the aligned rule):
    // 2T - 1 on the first chunk = (2 num - div) / div
    FrameCount grown(bool aligned) const {
        FrameCount g = *this;
        g.mul = 2 * mul;
        g.add_first = 2 * add_first - (aligned ? 0 : div);
        g.add_rest = 2 * add_rest;
        return g;
    }
    // temporal stride 2: (T + 1) / 2 on the first chunk with the first frame on
    // its own (phase 0), else T / 2
    FrameCount halved(bool aligned) const {
        FrameCount g = *this;
        g.div = 2 * div;
        if (!aligned) g.add_first = add_first + div;
        return g;
    }
};

struct Slot {
    bool defined = false;
    int c = 0, h = 0, w = 0;
    FrameCount tc;
    size_t bytes = 0;
    void* ptr = nullptr;  // intermediates only
    int writer = -1;      // first op that writes it (-1: the input x or the residual argument)
    bool grouped = false; // written inside the frame-batched group: holds one batch
    FrameCount rel;       // grouped (and the slots the group reads): frames per batch of the group input
};

struct OpRt {
    int kind = 0;
    int cin = 0, cout = 0, kt = 1, kh = 1, kw = 1, up_s = 1, up_t = 1, tpad = 0;
    int stride_s = 1, stride_t = 1;
    int src = -1, res = -1, out = -1, act_out = -1;
    int norm_src = -1;      // act computed by a separate norm pass reading this slot
    int h_in = 0, w_in = 0, h_out = 0, w_out = 0;
    void* wpk = nullptr;    // packed (bf16) or copied (f32) weights
    float* bias = nullptr;
    float* gamma = nullptr;
    size_t cache_off = 0, cache_bytes = 0;
    int ntile = 0, nblocks = 0, kchunks = 0, family = 1;
    bool fused_act = false;
    bool out_u8 = false;  // y as 8-bit codes
    // This op also writes the cache of op cache_to (a later conv whose input it
    // produces) when the pass has enough frames: from its conv kernel or its
    // norm pass (cache_norm), the result v or the act (cache_act).
    int cache_to = -1;
    bool cache_norm = false, cache_act = false;
};

}  // namespace

struct cc3d_plan {
    uint32_t magic = kPlanMagic;
    int device = 0;
    int dtype = CC3D_BF16;
    int elem = 2;
    int cin = 0, h = 0, w = 0;
    int max_t = 1;
    int y_elem = 2;  // bytes per element of y (1 with 8-bit output)
    bool grow_aligned = false;  // CC3D_GROW_ALIGNED: the first chunk grows every frame
    int batch_from = 0;         // frame-batched group: ops batch_from .. n_ops-1 ...
    int frame_batch = 0;        // ... run over batches of this many frames of the group input (0: off)
    FrameCount g_in;            // frame count of the group input (the slots it reads from before it)
    float eps = 1e-6f;
    std::vector<Slot> slots;
    std::vector<OpRt> ops;
    size_t state_bytes = kAlign;
    size_t device_bytes = 0;
    bool uses_aux = false;
    std::vector<void*> allocs;

    // live event timing (cc3d_profile_*); mutable: forward_chunk takes a const plan
    struct Pending {
        hipEvent_t start, stop;
        double flops, bytes;
    };
    struct ProfPart {
        std::string kernel;
        int64_t launches = 0;
        double ms = 0.0, flops = 0.0, bytes = 0.0;
        std::vector<Pending> pending;
    };
    mutable bool prof_on = false;
    mutable std::vector<ProfPart> prof;  // ops.size() * 3
    mutable std::vector<hipEvent_t> event_pool;
};

namespace {

int test_fail_alloc_at()
{
    const char* s = getenv("CC3D_TEST_FAIL_ALLOC");
    return s ? atoi(s) : 0;
}

// Device memory for a plan: hipMalloc'd blocks the plan owns, or (arena mode)
// 256-byte-aligned ranges of a caller-given arena, reserved in order and never
// freed (the no-alloc entry point's scratch).
struct Allocator {
    cc3d_plan* p;
    int count = 0;
    int fail_at;
    char* arena = nullptr;
    size_t arena_cap = 0, arena_used = 0;
    explicit Allocator(cc3d_plan* plan) : p(plan), fail_at(test_fail_alloc_at()) {}
    Allocator(cc3d_plan* plan, void* base, size_t cap) : p(plan), fail_at(0), arena((char*)base), arena_cap(cap) {}
    cc3d_status alloc(void** out, size_t bytes, const char* what) {
        ++count;
        if (arena) {
            const size_t need = align_up(bytes ? bytes : 1);
            if (arena_used + need > arena_cap)
                return fail(CC3D_ENOMEM,
                            "this conv needs more than the %zu bytes of the no-alloc scratch (%s: %zu bytes "
                            "after %zu already reserved); use cc3d_plan_create / cc3d_forward_chunk",
                            arena_cap, what, bytes, arena_used);
            *out = arena + arena_used;
            arena_used += need;
            p->device_bytes += bytes;
            return CC3D_OK;
        }
        void* d = nullptr;
        if (fail_at > 0 && count == fail_at)
            return fail(CC3D_ENOMEM, "allocation %d (%s, %zu bytes) failed (injected by CC3D_TEST_FAIL_ALLOC)",
                        count, what, bytes);
        hipError_t e = hipMalloc(&d, bytes ? bytes : 1);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(CC3D_ENOMEM, "hipMalloc of %zu bytes for %s failed: %s", bytes, what,
                        hipGetErrorString(e));
        }
        p->allocs.push_back(d);
        p->device_bytes += bytes;
        *out = d;
        return CC3D_OK;
    }
};

void release(cc3d_plan* p)
{
    if (!p) return;
    int cur = 0;
    bool switched = false;
    if (hipGetDevice(&cur) == hipSuccess && cur != p->device) switched = hipSetDevice(p->device) == hipSuccess;
    for (void* d : p->allocs) (void)hipFree(d);
    p->allocs.clear();
    for (auto& part : p->prof)
        for (auto& e : part.pending) {
            (void)hipEventDestroy(e.start);
            (void)hipEventDestroy(e.stop);
        }
    for (hipEvent_t e : p->event_pool) (void)hipEventDestroy(e);
    if (switched) (void)hipSetDevice(cur);
    p->magic = 0;
    delete p;
}

bool valid_dtype(int d) { return d == CC3D_F32 || d == CC3D_BF16; }
bool valid_slot_ref(int s) { return s >= 0 && s < CC3D_MAX_SLOTS; }
const char* kind_name(int k) { return k == CC3D_OP_CONV ? "CONV" : "NORM_ACT"; }

cc3d_status build_group(const cc3d_stack_desc* d, cc3d_plan* p);

// Geometry and wiring checks, no device work.
cc3d_status build_graph(const cc3d_stack_desc* d, cc3d_plan* p)
{
    if (!d) return fail(CC3D_EINVAL, "stack desc is NULL");
    if (!valid_dtype(d->dtype)) return fail(CC3D_EDTYPE, "dtype %d not accepted (0 = F32, 1 = BF16)", d->dtype);
    if (d->cin <= 0 || d->h <= 0 || d->w <= 0)
        return fail(CC3D_ESHAPE, "input cin=%d h=%d w=%d: all must be >= 1", d->cin, d->h, d->w);
    if (d->max_chunk_t < 1 || d->max_chunk_t > 4096)
        return fail(CC3D_ESHAPE, "max_chunk_t=%d not in [1, 4096]", d->max_chunk_t);
    if (!(d->eps >= 0.0f) || d->eps > 1.0f) return fail(CC3D_EINVAL, "eps=%g not in [0, 1]", (double)d->eps);
    if (d->n_ops < 1 || d->n_ops > CC3D_MAX_OPS)
        return fail(CC3D_EINVAL, "n_ops=%d not in [1, %d]", d->n_ops, CC3D_MAX_OPS);
    if (!d->ops) return fail(CC3D_EINVAL, "ops is NULL");
    if (d->fold_upsample != 0 && d->fold_upsample != 1)
        return fail(CC3D_EINVAL, "fold_upsample=%d not accepted (0 or 1)", d->fold_upsample);
    if (d->grow != CC3D_GROW_ONCE && d->grow != CC3D_GROW_ALIGNED)
        return fail(CC3D_EINVAL, "grow=%d not accepted (0 = CC3D_GROW_ONCE, 1 = CC3D_GROW_ALIGNED)", d->grow);
    const bool bf16 = d->dtype == CC3D_BF16;
    if (bf16 && d->cin % 8 != 0)
        return fail(CC3D_ESHAPE, "bf16 input channels %d: must be a multiple of 8", d->cin);

    p->dtype = d->dtype;
    p->elem = bf16 ? 2 : 4;
    p->cin = d->cin;
    p->h = d->h;
    p->w = d->w;
    p->max_t = d->max_chunk_t;
    p->eps = d->eps;
    p->grow_aligned = d->grow == CC3D_GROW_ALIGNED;
    p->slots.assign(CC3D_MAX_SLOTS, Slot());
    Slot& x = p->slots[CC3D_SLOT_X];
    x.defined = true;
    x.c = d->cin;
    x.h = d->h;
    x.w = d->w;
    x.tc.mul = 1;

    auto define = [&](int slot, int c, int h, int w, const FrameCount& tc, int op) -> cc3d_status {
        if (slot == CC3D_SLOT_X || slot == CC3D_SLOT_AUX)
            return fail(CC3D_EINVAL, "op %d writes slot %d (the input x or the residual argument)", op, slot);
        Slot& s = p->slots[slot];
        if (s.defined) {
            if (s.c != c || s.h != h || s.w != w || !(s.tc == tc))
                return fail(CC3D_ESHAPE, "op %d writes slot %d as %dx%dx%d but it holds %dx%dx%d", op, slot, c, h,
                            w, s.c, s.h, s.w);
            return CC3D_OK;
        }
        s.defined = true;
        s.c = c;
        s.h = h;
        s.w = w;
        s.tc = tc;
        s.writer = op;
        return CC3D_OK;
    };

    size_t cache_off = 0;
    int y_u8_seen = -1;  // -1: no op writes y yet; else whether it is 8-bit
    for (int i = 0; i < d->n_ops; ++i) {
        const cc3d_op_desc& o = d->ops[i];
        OpRt r;
        r.kind = o.kind;
        if (o.kind != CC3D_OP_CONV && o.kind != CC3D_OP_NORM_ACT)
            return fail(CC3D_EINVAL, "op %d: kind %d not accepted (0 = CONV, 1 = NORM_ACT)", i, o.kind);
        if (!valid_slot_ref(o.src) || !p->slots[o.src].defined)
            return fail(CC3D_EINVAL, "op %d: src slot %d is not defined by an earlier op", i, o.src);
        for (int s : {o.res, o.out, o.act_out})
            if (s != CC3D_SLOT_NONE && !valid_slot_ref(s))
                return fail(CC3D_EINVAL, "op %d: slot %d not in [0, %d) or -1", i, s, CC3D_MAX_SLOTS);
        if (o.out == CC3D_SLOT_NONE && o.act_out == CC3D_SLOT_NONE)
            return fail(CC3D_EINVAL, "op %d: neither out nor act_out is set", i);
        if (o.out != CC3D_SLOT_NONE && o.out == o.act_out)
            return fail(CC3D_EINVAL, "op %d: out and act_out are the same slot %d", i, o.out);
        if (o.out == o.src || o.act_out == o.src || (o.res != CC3D_SLOT_NONE && (o.res == o.out || o.res == o.act_out)))
            return fail(CC3D_EINVAL, "op %d: an output slot is also an input slot", i);
        const Slot src = p->slots[o.src];
        r.src = o.src;
        r.res = o.res;
        r.out = o.out;
        r.act_out = o.act_out;
        r.cin = src.c;
        r.h_in = src.h;
        r.w_in = src.w;
        FrameCount tc_out = src.tc;
        if (o.kind == CC3D_OP_CONV) {
            if (o.kt < 1 || o.kt > 3 || o.kh < 1 || o.kh > 3 || o.kw < 1 || o.kw > 3 || o.kh % 2 == 0 || o.kw % 2 == 0)
                return fail(CC3D_ESHAPE, "op %d: kernel %dx%dx%d; accepted: kt 1..3, kh and kw 1 or 3", i, o.kt,
                            o.kh, o.kw);
            if ((o.up_s != 1 && o.up_s != 2) || (o.up_t != 1 && o.up_t != 2))
                return fail(CC3D_ESHAPE, "op %d: up_s=%d up_t=%d; accepted 1 or 2", i, o.up_s, o.up_t);
            if (o.stride_s < 0 || o.stride_s > 2 || o.stride_t < 0 || o.stride_t > 2)
                return fail(CC3D_ESHAPE, "op %d: stride_s=%d stride_t=%d; accepted 1 or 2 (0 reads as 1)", i,
                            o.stride_s, o.stride_t);
            r.stride_s = o.stride_s == 2 ? 2 : 1;
            r.stride_t = o.stride_t == 2 ? 2 : 1;
            if ((r.stride_s == 2 && o.up_s == 2) || (r.stride_t == 2 && o.up_t == 2))
                return fail(CC3D_ESHAPE, "op %d: a conv either upsamples or strides along an axis (up_s=%d "
                            "stride_s=%d, up_t=%d stride_t=%d)", i, o.up_s, r.stride_s, o.up_t, r.stride_t);
            if ((r.stride_s == 2 || r.stride_t == 2) && o.out_u8)
                return fail(CC3D_EINVAL, "op %d: 8-bit output is not taken by a strided conv", i);
            if (o.tpad != CC3D_TPAD_REPLICATE && o.tpad != CC3D_TPAD_ZERO)
                return fail(CC3D_EINVAL, "op %d: tpad %d not accepted (0 = REPLICATE, 1 = ZERO)", i, o.tpad);
            if (o.cout < 1 || o.cout > 4096) return fail(CC3D_ESHAPE, "op %d: cout=%d not in [1, 4096]", i, o.cout);
            if (!o.w) return fail(CC3D_EINVAL, "op %d: weights are NULL", i);
            if (bf16) {
                if (r.cin % 8 != 0)
                    return fail(CC3D_ESHAPE, "op %d: bf16 conv input channels %d: must be a multiple of 8", i, r.cin);
                if (o.kh != o.kw) return fail(CC3D_ESHAPE, "op %d: bf16 conv needs kh == kw (got %d, %d)", i, o.kh, o.kw);
                if ((int64_t)r.h_in * r.w_in * r.cin >= ((int64_t)1 << 30))
                    return fail(CC3D_ESHAPE, "op %d: input frame of %lld elements; accepted below 2^30", i,
                                (long long)r.h_in * r.w_in * r.cin);
                if (!cc3d::bf16_conv_supported(o.cout, o.kh, o.kw, o.up_s))
                    return fail(CC3D_ESHAPE, "op %d: bf16 conv cout=%d k=%d up_s=%d has no kernel", i, o.cout, o.kh,
                                o.up_s);
            }
            if ((int64_t)r.h_in * o.up_s > 65535 || (int64_t)r.w_in * o.up_s > 65535)
                return fail(CC3D_ESHAPE, "op %d: output frame %dx%d exceeds 65535", i, r.h_in * o.up_s, r.w_in * o.up_s);
            r.cout = o.cout;
            r.kt = o.kt;
            r.kh = o.kh;
            r.kw = o.kw;
            r.up_s = o.up_s;
            r.up_t = o.up_t;
            r.tpad = o.tpad;
            r.h_out = r.stride_s == 2 ? (r.h_in + 1) / 2 : r.h_in * o.up_s;
            r.w_out = r.stride_s == 2 ? (r.w_in + 1) / 2 : r.w_in * o.up_s;
            if (o.up_t == 2) tc_out = src.tc.grown(p->grow_aligned);
            if (r.stride_t == 2) tc_out = src.tc.halved(p->grow_aligned);
            r.cache_off = cache_off;
            r.cache_bytes = (size_t)(o.kt - 1) * r.h_in * r.w_in * r.cin * p->elem;
            cache_off += align_up(r.cache_bytes);
            if (bf16) {
                cc3d::bf16_conv_tiling(o.cout, &r.ntile, &r.nblocks);
                r.kchunks = (r.cin + 31) / 32;
                const int plain = o.act_out == CC3D_SLOT_NONE && !o.out_u8;
                r.family = cc3d::bf16_conv_family(o.cout, r.cin, o.kt, o.kh, o.kw, o.up_s, plain,
                                                  d->fold_upsample && !o.out_u8);
                if (r.stride_s == 2 || r.stride_t == 2) {
                    // 3x3 spatial stride 2 in 96/128-channel blocks: the register-blocked
                    // kernel's strided tile; any other strided conv: the generic kernel
                    r.family = (r.family == 2 && r.stride_s == 2) ? 2 : 1;
                    // 8 input channels (pixels padded to 8): the temporal taps fold into
                    // one 32-channel K step
                    if (r.family == 2 && r.cin == 8 && o.kt <= 3) r.family = 6;
                    // output channels a multiple of 192: the strided tile in 192-channel
                    // blocks (twice the MFMAs per LDS fragment read of the 96-channel one)
                    if (r.family == 2 && o.cout % 192 == 0) {
                        r.family = 7;
                        r.ntile = 192;
                        r.nblocks = o.cout / 192;
                    }
                }
                if (r.family == 4) cc3d::pw_conv_tiling(o.cout, &r.ntile, &r.nblocks);
            }
        } else {
            r.cout = r.cin;
            r.h_out = r.h_in;
            r.w_out = r.w_in;
            if (r.cin % 4 != 0 || r.cin > 512)
                return fail(CC3D_ESHAPE, "op %d: NORM_ACT channels %d; accepted a multiple of 4 up to 512", i, r.cin);
        }
        if (o.act_out != CC3D_SLOT_NONE) {
            if (!o.gamma) return fail(CC3D_EINVAL, "op %d: act_out is set but gamma is NULL", i);
            if (r.cout % 4 != 0 || r.cout > 512)
                return fail(CC3D_ESHAPE, "op %d: act over %d channels; accepted a multiple of 4 up to 512", i, r.cout);
        }
        if (o.out_u8) {
            if (o.kind != CC3D_OP_CONV || o.out != CC3D_SLOT_Y || o.act_out != CC3D_SLOT_NONE)
                return fail(CC3D_EINVAL, "op %d: out_u8 is accepted on a CONV op that writes only the output slot", i);
            if (!bf16) return fail(CC3D_EDTYPE, "op %d: 8-bit output needs a bf16 plan", i);
            if (r.family == 2)
                return fail(CC3D_ESHAPE,
                            "op %d: 8-bit output is not written by the 3x3 kernel for 96/128-channel blocks "
                            "(cout=%d); accepted: cout <= 64, or the 3x3x3 head to <= 3 channels", i,
                            r.cout);
            r.out_u8 = true;
        }
        if (o.out == CC3D_SLOT_Y && (y_u8_seen >= 0) && (y_u8_seen != (o.out_u8 ? 1 : 0)))
            return fail(CC3D_EINVAL, "op %d: the output slot is written both as 8-bit codes and as the plan dtype", i);
        if (o.out == CC3D_SLOT_Y) y_u8_seen = o.out_u8 ? 1 : 0;
        if (o.res != CC3D_SLOT_NONE) {
            if (o.res == CC3D_SLOT_AUX && !p->slots[CC3D_SLOT_AUX].defined) {
                Slot& a = p->slots[CC3D_SLOT_AUX];
                a.defined = true;
                a.c = r.cout;
                a.h = r.h_out;
                a.w = r.w_out;
                a.tc = tc_out;
            }
            const Slot& rs = p->slots[o.res];
            if (!rs.defined) return fail(CC3D_EINVAL, "op %d: residual slot %d is not defined", i, o.res);
            if (rs.c == r.cout && rs.h == r.h_out && rs.w == r.w_out && !(rs.tc == tc_out))
                return fail(CC3D_ESHAPE, "op %d: residual slot %d has another frame count than the result "
                            "(one is grown in time)", i, o.res);
            if (rs.c != r.cout || rs.h != r.h_out || rs.w != r.w_out)
                return fail(CC3D_ESHAPE, "op %d: residual slot %d is %dx%dx%d, the result is %dx%dx%d", i, o.res, rs.c,
                            rs.h, rs.w, r.cout, r.h_out, r.w_out);
            if (o.res == CC3D_SLOT_AUX) p->uses_aux = true;
        }
        if (o.out != CC3D_SLOT_NONE) {
            cc3d_status st = define(o.out, r.cout, r.h_out, r.w_out, tc_out, i);
            if (st != CC3D_OK) return st;
        }
        if (o.act_out != CC3D_SLOT_NONE) {
            cc3d_status st = define(o.act_out, r.cout, r.h_out, r.w_out, tc_out, i);
            if (st != CC3D_OK) return st;
        }
        // The act is fused into the bf16 conv when one workgroup holds every
        // output channel; otherwise a norm pass reads the stored result.
        if (o.kind == CC3D_OP_CONV && o.act_out != CC3D_SLOT_NONE)
            r.fused_act = bf16 && r.nblocks == 1;
        p->ops.push_back(r);
    }
    if (!p->slots[CC3D_SLOT_Y].defined) return fail(CC3D_EINVAL, "no op writes the output slot %d", CC3D_SLOT_Y);
    p->y_elem = y_u8_seen == 1 ? 1 : p->elem;
    for (const OpRt& r : p->ops)
        if (r.kind == CC3D_OP_NORM_ACT && (r.out == CC3D_SLOT_Y || r.act_out == CC3D_SLOT_Y) && p->y_elem == 1)
            return fail(CC3D_EINVAL, "the output slot is written both as 8-bit codes and as the plan dtype");
    p->state_bytes = cache_off < kAlign ? kAlign : cache_off;
    return build_group(d, p);
}

// Frame-batched group (frame_batch > 0): ops batch_from.. run over batches of
// frame_batch frames of the group input, the slots they read from before the
// group, which must all have one frame count.  Their own slots hold one batch;
// frame counts inside the group are kept relative to the group input.
cc3d_status build_group(const cc3d_stack_desc* d, cc3d_plan* p)
{
    if (d->frame_batch < 0 || d->frame_batch > 4096)
        return fail(CC3D_EINVAL, "frame_batch=%d not in [0, 4096]", d->frame_batch);
    if (d->frame_batch == 0) return CC3D_OK;
    const int n = (int)p->ops.size();
    if (d->batch_from < 0 || d->batch_from >= n)
        return fail(CC3D_EINVAL, "batch_from=%d not in [0, %d) (the op list)", d->batch_from, n);
    p->batch_from = d->batch_from;
    p->frame_batch = d->frame_batch;
    bool have = false;
    for (int i = d->batch_from; i < n; ++i) {
        const OpRt& r = p->ops[i];
        if (r.stride_s != 1 || r.stride_t != 1)
            return fail(CC3D_EINVAL, "op %d: a strided conv is not taken inside the frame-batched group", i);
        for (int sl : {r.src, r.res}) {
            if (sl == CC3D_SLOT_NONE) continue;
            if (sl == CC3D_SLOT_AUX)
                return fail(CC3D_EINVAL, "op %d of the frame-batched group reads the residual argument", i);
            Slot& in = p->slots[sl];
            if (in.writer >= d->batch_from) continue;  // written inside the group
            if (!have) {
                p->g_in = in.tc;
                have = true;
            } else if (!(in.tc == p->g_in)) {
                return fail(CC3D_ESHAPE, "the frame-batched group reads slots of different frame counts (op %d, slot %d)",
                            i, sl);
            }
            in.rel = FrameCount();
            in.rel.mul = 1;
        }
        for (int sl : {r.out, r.act_out}) {
            if (sl == CC3D_SLOT_NONE) continue;
            if (p->slots[sl].writer < d->batch_from)
                return fail(CC3D_EINVAL, "op %d of the frame-batched group writes slot %d, also written before the group",
                            i, sl);
        }
    }
    if (!have) return fail(CC3D_EINVAL, "the frame-batched group reads nothing computed before it");
    if (p->slots[CC3D_SLOT_Y].writer < d->batch_from)
        return fail(CC3D_EINVAL, "the output slot must be written inside the frame-batched group");
    for (int i = d->batch_from; i < n; ++i) {
        const OpRt& r = p->ops[i];
        const FrameCount rel_in = p->slots[r.src].rel;
        const FrameCount rel_out = (r.kind == CC3D_OP_CONV && r.up_t == 2) ? rel_in.grown(p->grow_aligned) : rel_in;
        for (int sl : {r.out, r.act_out}) {
            if (sl == CC3D_SLOT_NONE) continue;
            p->slots[sl].grouped = true;
            p->slots[sl].rel = rel_out;
        }
    }
    return CC3D_OK;
}

// Slots an unfused act needs: the conv result must be stored somewhere.
cc3d_status assign_norm_temps(cc3d_plan* p)
{
    for (OpRt& r : p->ops) {
        if (r.kind != CC3D_OP_CONV || r.act_out == CC3D_SLOT_NONE || r.fused_act) continue;
        if (r.out != CC3D_SLOT_NONE) {
            r.norm_src = r.out;
            continue;
        }
        int tmp = -1;
        for (int s = CC3D_MAX_SLOTS - 1; s > CC3D_SLOT_AUX; --s)
            if (!p->slots[s].defined) {
                tmp = s;
                break;
            }
        if (tmp < 0) return fail(CC3D_EINVAL, "no free slot left for an unfused act (all %d in use)", CC3D_MAX_SLOTS);
        Slot& t = p->slots[tmp];
        const Slot& a = p->slots[r.act_out];
        t = a;
        t.defined = true;
        r.norm_src = tmp;
    }
    return CC3D_OK;
}

// A conv's cache holds the last kt-1 frames of its window; when its input is a
// slot an earlier op of the same pass writes and the conv does not grow time,
// those are the slot's last kt-1 frames (whenever the pass has that many), so
// the writing op can store them into the cache as it produces them instead of
// a copy kernel reading them back.  Pairs each such conv with its input's
// writer: the writer's conv kernel where it is one of the register-blocked
// families (which take a cache destination) or its norm pass.  Ops of a
// frame-batched group keep the copy (a batch continues its caches in place).
void pair_cache_writers(cc3d_plan* p)
{
    const int n = (int)p->ops.size();
    const int g0 = p->frame_batch > 0 ? p->batch_from : n;
    for (int j = 0; j < n && j < g0; ++j) {
        const OpRt& c = p->ops[j];
        if (c.kind != CC3D_OP_CONV || c.kt < 2 || c.up_t != 1 || c.src <= CC3D_SLOT_AUX) continue;
        int i = j - 1;
        for (; i >= 0; --i) {
            const OpRt& w = p->ops[i];
            if (w.out == c.src || w.act_out == c.src) break;
        }
        if (i < 0) continue;
        OpRt& w = p->ops[i];
        if (w.cache_to >= 0) continue;  // one cache per writer
        const bool act = w.act_out == c.src;
        bool norm;
        if (w.kind == CC3D_OP_NORM_ACT) norm = true;
        else if (act) norm = !w.fused_act;
        else norm = false;  // the conv kernel writes its result slot
        if (!norm && !(p->dtype == CC3D_BF16 && (w.family == 2 || w.family == 5 || w.family == 6 ||
                                                  w.family == 7))) continue;
        w.cache_to = j;
        w.cache_norm = norm;
        w.cache_act = act;
    }
}

cc3d_status hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return CC3D_OK;
    (void)hipGetLastError();
    return fail(CC3D_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) {
            ok = false;
            prev = -1;
            return;
        }
        if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// Device memory of a plan and its contents: first every block is reserved (so
// a plan that does not fit fails before any device work), then the weights are
// repacked or copied and bias/gain copied on `stream`.  `sync`: wait for that
// work (plan creation; the no-alloc path does not).
cc3d_status materialise(const cc3d_stack_desc* d, cc3d_plan* p, hipStream_t stream, Allocator& al, bool sync)
{
    // intermediate slots
    for (int s = CC3D_SLOT_AUX + 1; s < CC3D_MAX_SLOTS; ++s) {
        Slot& sl = p->slots[s];
        if (!sl.defined) continue;
        const int64_t tmax = sl.grouped ? sl.rel.bound(p->frame_batch) : sl.tc.bound(p->max_t);
        sl.bytes = (size_t)tmax * sl.h * sl.w * sl.c * p->elem;
        cc3d_status st = al.alloc(&sl.ptr, sl.bytes, "an intermediate slot");
        if (st != CC3D_OK) return st;
    }
    for (size_t i = 0; i < p->ops.size(); ++i) {
        OpRt& r = p->ops[i];
        const cc3d_op_desc& o = d->ops[i];
        cc3d_status st = CC3D_OK;
        if (r.kind == CC3D_OP_CONV) {
            const size_t wbytes = p->dtype == CC3D_BF16
                                      ? cc3d::bf16_packed_elems(r.cout, r.cin, r.kt, r.kh, r.kw, r.family) * 2
                                      : (size_t)r.cout * r.cin * r.kt * r.kh * r.kw * p->elem;
            st = al.alloc(&r.wpk, wbytes, p->dtype == CC3D_BF16 ? "packed weights" : "weights");
            if (st != CC3D_OK) return st;
            if (o.bias) {
                void* b = nullptr;
                if ((st = al.alloc(&b, (size_t)r.cout * 4, "bias")) != CC3D_OK) return st;
                r.bias = (float*)b;
            }
        }
        if (r.act_out != CC3D_SLOT_NONE) {
            void* g = nullptr;
            if ((st = al.alloc(&g, (size_t)r.cout * 4, "gamma")) != CC3D_OK) return st;
            r.gamma = (float*)g;
        }
    }
    for (size_t i = 0; i < p->ops.size(); ++i) {
        const OpRt& r = p->ops[i];
        const cc3d_op_desc& o = d->ops[i];
        cc3d_status st = CC3D_OK;
        if (r.kind == CC3D_OP_CONV) {
            if (p->dtype == CC3D_BF16)
                st = hip_status(cc3d::launch_pack_bf16(o.w, r.wpk, r.cout, r.cin, r.kt, r.kh, r.kw, r.family, stream),
                                "weight repack launch");
            else
                st = hip_status(hipMemcpyAsync(r.wpk, o.w, (size_t)r.cout * r.cin * r.kt * r.kh * r.kw * p->elem,
                                               hipMemcpyDeviceToDevice, stream),
                                "weight copy");
            if (st != CC3D_OK) return st;
            if (o.bias) {
                st = hip_status(hipMemcpyAsync(r.bias, o.bias, (size_t)r.cout * 4, hipMemcpyDeviceToDevice, stream),
                                "bias copy");
                if (st != CC3D_OK) return st;
            }
        }
        if (r.act_out != CC3D_SLOT_NONE) {
            st = hip_status(hipMemcpyAsync(r.gamma, o.gamma, (size_t)r.cout * 4, hipMemcpyDeviceToDevice, stream),
                            "gamma copy");
            if (st != CC3D_OK) return st;
        }
    }
    return sync ? hip_status(hipStreamSynchronize(stream), "plan set-up") : CC3D_OK;
}

std::string conv_kernel_name(const cc3d_plan* p, const OpRt& r);

// The plan's graph, slots and op table, with no device work.
cc3d_status build_plan(const cc3d_stack_desc* d, cc3d_plan* p)
{
    cc3d_status st = build_graph(d, p);
    if (st != CC3D_OK) return st;
    st = assign_norm_temps(p);
    if (st != CC3D_OK) return st;
    pair_cache_writers(p);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    p->device = dev;
    return CC3D_OK;
}

void name_kernels(cc3d_plan* p)
{
    p->prof.assign(p->ops.size() * 3, cc3d_plan::ProfPart());
    const char* norm_name = p->dtype == CC3D_BF16 ? "norm_act_bf16" : "norm_act_f32";
    for (size_t i = 0; i < p->ops.size(); ++i) {
        const OpRt& r = p->ops[i];
        if (r.kind == CC3D_OP_CONV) {
            p->prof[i * 3 + 0].kernel = conv_kernel_name(p, r);
            if (r.act_out != CC3D_SLOT_NONE && !r.fused_act) p->prof[i * 3 + 1].kernel = norm_name;
            if (r.kt > 1) p->prof[i * 3 + 2].kernel = "cache_update";
        } else {
            p->prof[i * 3 + 0].kernel = norm_name;
        }
    }
}

cc3d_status noalloc_scratch(int device, void** out);

cc3d_status create_common(const cc3d_stack_desc* d, void* stream, cc3d_plan** out)
{
    if (!out) return fail(CC3D_EINVAL, "out is NULL");
    *out = nullptr;
    cc3d_plan* p = new (std::nothrow) cc3d_plan();
    if (!p) return fail(CC3D_ENOMEM, "host allocation of the plan failed");
    cc3d_status st = build_plan(d, p);
    if (st == CC3D_OK) {
        // set-up on this device: the no-alloc entry point's scratch address too
        void* unused = nullptr;
        st = noalloc_scratch(p->device, &unused);
    }
    if (st == CC3D_OK) {
        Allocator al(p);
        st = materialise(d, p, (hipStream_t)stream, al, true);
    }
    if (st != CC3D_OK) {
        release(p);
        return st;
    }
    name_kernels(p);
    *out = p;
    clear_err();
    return CC3D_OK;
}

bool plan_ok(const cc3d_plan* p) { return p && p->magic == kPlanMagic; }

// A chunk of t_chunk frames must leave every slot a whole frame count (strided
// convs halve it: see FrameCount).
cc3d_status check_frames(const cc3d_plan* p, int t_chunk, bool first)
{
    for (int s = 0; s < CC3D_MAX_SLOTS; ++s) {
        const Slot& sl = p->slots[s];
        if (!sl.defined || sl.tc.whole(t_chunk, first)) continue;
        return fail(CC3D_ESHAPE,
                    "t_chunk=%d (%s chunk) leaves op %d's output a fractional frame count: a temporal stride of 2 "
                    "needs an %s number of frames there",
                    t_chunk, first ? "first" : "later", sl.writer,
                    (first && !p->grow_aligned) ? "odd" : "even");
    }
    return CC3D_OK;
}

cc3d_status check_ptr(const void* ptr, int device, const char* what)
{
    hipPointerAttribute_t at;
    hipError_t e = hipPointerGetAttributes(&at, ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(CC3D_EDEVICE, "%s (%p) is not memory known to HIP: %s", what, ptr, hipGetErrorString(e));
    }
    if (at.type == hipMemoryTypeHost || at.type == hipMemoryTypeUnregistered)
        return fail(CC3D_EDEVICE, "%s (%p) is host memory; a device pointer is required", what, ptr);
    if (at.type == hipMemoryTypeDevice && at.device != device)
        return fail(CC3D_EDEVICE, "%s (%p) is on device %d, the plan on device %d", what, ptr, at.device, device);
    return CC3D_OK;
}

hipEvent_t take_event(const cc3d_plan* p)
{
    if (!p->event_pool.empty()) {
        hipEvent_t e = p->event_pool.back();
        p->event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return e;
}

// Event pair around one launch; inactive when profiling is off or events run out.
struct ProfScope {
    const cc3d_plan* p;
    size_t slot;
    hipStream_t s;
    hipEvent_t a = nullptr, b = nullptr;
    double flops, bytes;
    ProfScope(const cc3d_plan* plan, size_t op, int part, hipStream_t st, double f, double by)
        : p(plan), slot(op * 3 + part), s(st), flops(f), bytes(by) {
        if (!p->prof_on) return;
        a = take_event(p);
        b = take_event(p);
        if (a && b) {
            (void)hipEventRecord(a, s);
        } else {
            if (a) p->event_pool.push_back(a);
            if (b) p->event_pool.push_back(b);
            a = b = nullptr;
        }
    }
    ~ProfScope() {
        if (!a) return;
        (void)hipEventRecord(b, s);
        p->prof[slot].pending.push_back({a, b, flops, bytes});
    }
};

std::string conv_kernel_name(const cc3d_plan* p, const OpRt& r)
{
    char buf[64];
    if (p->dtype == CC3D_BF16 && r.family == 3)
        snprintf(buf, sizeof buf, "conv_bf16_head_up%d_k%d_c%d", r.up_s, r.kh, r.cout);
    else if (p->dtype == CC3D_BF16 && r.family == 5)
        snprintf(buf, sizeof buf, "conv_bf16_phase_up%d_k%d_n%d", r.up_s, r.kh, r.ntile);
    else if (p->dtype == CC3D_BF16 && r.family == 4)
        snprintf(buf, sizeof buf, "conv_bf16_pw_up%d_kt%d_n%d", r.up_s, r.kt, r.ntile);
    else if (p->dtype == CC3D_BF16 && (r.stride_s > 1 || r.stride_t > 1))
        snprintf(buf, sizeof buf, "conv_bf16%s_s%dt%d_k%d_n%d",
                 r.family == 6 ? "_v2tf" : ((r.family == 2 || r.family == 7) ? "_v2" : ""), r.stride_s, r.stride_t,
                 r.kh, r.ntile);
    else if (p->dtype == CC3D_BF16)
        snprintf(buf, sizeof buf, "conv_bf16%s_up%d_k%d_n%d", r.family == 2 ? "_v2" : "", r.up_s, r.kh,
                 r.ntile);
    else
        snprintf(buf, sizeof buf, "conv_f32");
    return buf;
}

// The one-op stack descriptor of a single-conv descriptor.
cc3d_status conv_stack_desc(const cc3d_conv_desc* d, const void* w, const float* bias, const float* gamma,
                            cc3d_op_desc* op, cc3d_stack_desc* sd)
{
    if (!d) return fail(CC3D_EINVAL, "conv desc is NULL");
    if (d->epilogue & ~(CC3D_EPI_RESIDUAL | CC3D_EPI_ACT | CC3D_EPI_U8))
        return fail(CC3D_EINVAL, "epilogue flags 0x%x; accepted CC3D_EPI_RESIDUAL | CC3D_EPI_ACT | CC3D_EPI_U8",
                    d->epilogue);
    if ((d->epilogue & CC3D_EPI_ACT) && (d->epilogue & CC3D_EPI_U8))
        return fail(CC3D_EINVAL, "CC3D_EPI_U8 cannot be combined with CC3D_EPI_ACT");
    if (d->cin <= 0) return fail(CC3D_ESHAPE, "cin=%d must be >= 1", d->cin);
    memset(op, 0, sizeof *op);
    op->kind = CC3D_OP_CONV;
    op->cout = d->cout;
    op->kt = d->kt;
    op->kh = d->kh;
    op->kw = d->kw;
    op->up_s = d->up_s;
    op->up_t = d->up_t;
    op->tpad = d->tpad;
    op->src = CC3D_SLOT_X;
    op->res = (d->epilogue & CC3D_EPI_RESIDUAL) ? CC3D_SLOT_AUX : CC3D_SLOT_NONE;
    op->out = (d->epilogue & CC3D_EPI_ACT) ? CC3D_SLOT_NONE : CC3D_SLOT_Y;
    op->act_out = (d->epilogue & CC3D_EPI_ACT) ? CC3D_SLOT_Y : CC3D_SLOT_NONE;
    op->w = w;
    op->bias = bias;
    op->gamma = gamma;
    op->out_u8 = (d->epilogue & CC3D_EPI_U8) ? 1 : 0;
    op->stride_s = d->stride_s;
    op->stride_t = d->stride_t;
    memset(sd, 0, sizeof *sd);
    sd->dtype = d->dtype;
    sd->cin = d->cin;
    sd->h = d->h_in;
    sd->w = d->w_in;
    sd->max_chunk_t = d->max_chunk_t;
    sd->eps = d->eps;
    sd->grow = d->grow;
    sd->fold_upsample = d->fold_upsample;
    sd->n_ops = 1;
    sd->ops = op;
    return CC3D_OK;
}

// The no-alloc entry point's scratch: one array per device, in this file, of a
// fixed size (CC3D_NOALLOC_SCRATCH_BYTES), held until the process ends.  Its
// device address is looked up once per device (at the first plan creation or
// no-alloc call there) and kept: in host code the array's name is not a device
// address.
__device__ __align__(256) unsigned char scratch[CC3D_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

cc3d_status noalloc_scratch(int device, void** out)
{
    if (device < 0 || device >= kMaxDevices) return fail(CC3D_EDEVICE, "device %d not in [0, %d)", device, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(CC3D_EDEVICE, "hipGetSymbolAddress of the no-alloc scratch on device %d failed: %s", device,
                        hipGetErrorString(e));
        }
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return CC3D_OK;
}

// One chunk through a plan; with check_only, every argument check and nothing else.
cc3d_status forward_impl(const cc3d_plan* p, const void* x, int t_chunk, const cc3d_state* cache_in,
                         cc3d_state* cache_out, const void* residual, void* y, void* stream, bool check_only);

}  // namespace

extern "C" {

int cc3d_version(void) { return CC3D_VERSION; }

const char* cc3d_last_error(void) { return g_err; }

cc3d_status cc3d_stack_plan_create(const cc3d_stack_desc* desc, void* stream, cc3d_plan** out)
{
    return create_common(desc, stream, out);
}

cc3d_status cc3d_plan_create(const cc3d_conv_desc* d, const void* w, const float* bias, const float* gamma,
                             void* stream, cc3d_plan** out)
{
    if (out) *out = nullptr;
    cc3d_op_desc op;
    cc3d_stack_desc sd;
    cc3d_status st = conv_stack_desc(d, w, bias, gamma, &op, &sd);
    if (st != CC3D_OK) return st;
    return create_common(&sd, stream, out);
}

void cc3d_plan_destroy(cc3d_plan* plan)
{
    if (plan_ok(plan)) release(plan);
}

size_t cc3d_state_bytes(const cc3d_plan* plan) { return plan_ok(plan) ? plan->state_bytes : 0; }

size_t cc3d_plan_device_bytes(const cc3d_plan* plan) { return plan_ok(plan) ? plan->device_bytes : 0; }

int cc3d_output_elem_bytes(const cc3d_plan* plan) { return plan_ok(plan) ? plan->y_elem : 0; }

cc3d_status cc3d_output_shape(const cc3d_plan* p, int t_chunk, int first, int* c, int* t, int* h, int* w)
{
    if (!plan_ok(p)) return fail(CC3D_EINVAL, "plan is NULL or destroyed");
    if (t_chunk < 1 || t_chunk > p->max_t)
        return fail(CC3D_ESHAPE, "t_chunk=%d not in [1, %d]", t_chunk, p->max_t);
    cc3d_status st = check_frames(p, t_chunk, first != 0);
    if (st != CC3D_OK) return st;
    const Slot& y = p->slots[CC3D_SLOT_Y];
    if (c) *c = y.c;
    if (t) *t = (int)y.tc.eval(t_chunk, first != 0);
    if (h) *h = y.h;
    if (w) *w = y.w;
    clear_err();
    return CC3D_OK;
}

cc3d_status cc3d_reset(const cc3d_plan* p, cc3d_state* state, void* stream)
{
    if (!plan_ok(p)) return fail(CC3D_EINVAL, "plan is NULL or destroyed");
    if (!state) return fail(CC3D_EINVAL, "state is NULL");
    if (!state->arena) return fail(CC3D_EINVAL, "state arena is NULL");
    DeviceGuard g(p->device);
    if (!g.ok) return fail(CC3D_EDEVICE, "cannot make device %d current", p->device);
    cc3d_status st = check_ptr(state->arena, p->device, "state arena");
    if (st != CC3D_OK) return st;
    st = hip_status(cc3d::launch_fill_zero(state->arena, p->state_bytes, (hipStream_t)stream), "arena clear");
    if (st != CC3D_OK) return st;
    state->frames_seen = 0;
    clear_err();
    return CC3D_OK;
}

cc3d_status cc3d_forward_chunk(const cc3d_plan* p, const void* x, int t_chunk, const cc3d_state* cache_in,
                               cc3d_state* cache_out, const void* residual, void* y, void* stream)
{
    return forward_impl(p, x, t_chunk, cache_in, cache_out, residual, y, stream, false);
}

cc3d_status cc3d_conv_forward_noalloc(const cc3d_conv_desc* d, const void* w, const float* bias,
                                      const float* gamma, const void* x, int t_chunk,
                                      const cc3d_state* cache_in, cc3d_state* cache_out, const void* residual,
                                      void* y, void* stream)
{
    if (!w) return fail(CC3D_EINVAL, "w is NULL");
    if (!x) return fail(CC3D_EINVAL, "x is NULL");
    if (!y) return fail(CC3D_EINVAL, "y is NULL");
    cc3d_op_desc op;
    cc3d_stack_desc sd;
    cc3d_status st = conv_stack_desc(d, w, bias, gamma, &op, &sd);
    if (st != CC3D_OK) return st;
    // a plan on the host whose device memory is ranges of this device's scratch
    cc3d_plan plan;
    if ((st = build_plan(&sd, &plan)) != CC3D_OK) return st;
    if (t_chunk < 1 || t_chunk > plan.max_t)
        return fail(CC3D_ESHAPE, "t_chunk=%d not in [1, %d] (the descriptor's max_chunk_t)", t_chunk, plan.max_t);
    if ((st = check_ptr(w, plan.device, "w")) != CC3D_OK) return st;
    if (bias && (st = check_ptr(bias, plan.device, "bias")) != CC3D_OK) return st;
    if (gamma && (st = check_ptr(gamma, plan.device, "gamma")) != CC3D_OK) return st;
    void* base = nullptr;
    if ((st = noalloc_scratch(plan.device, &base)) != CC3D_OK) return st;
    // The chunk's arguments are checked first (forward_impl, check only); then
    // materialise reserves every block of the scratch before it launches
    // anything (a conv that does not fit fails there, before any device work),
    // repacks the weights into it, and the chunk runs, all on `stream`.
    Allocator al(&plan, base, CC3D_NOALLOC_SCRATCH_BYTES);
    plan.magic = kPlanMagic;
    st = forward_impl(&plan, x, t_chunk, cache_in, cache_out, residual, y, nullptr, true);
    if (st == CC3D_OK) st = materialise(&sd, &plan, (hipStream_t)stream, al, false);
    if (st == CC3D_OK) st = forward_impl(&plan, x, t_chunk, cache_in, cache_out, residual, y, stream, false);
    plan.magic = 0;
    return st;
}

cc3d_status cc3d_slot_shape(const cc3d_plan* p, int slot, int t_chunk, int first, int* c, int* t, int* h, int* w)
{
    if (!plan_ok(p)) return fail(CC3D_EINVAL, "plan is NULL or destroyed");
    if (slot < CC3D_SLOT_AUX || slot >= CC3D_MAX_SLOTS || !p->slots[slot].defined)
        return fail(CC3D_EINVAL, "slot %d is not an intermediate or residual slot of this plan", slot);
    if (t_chunk < 1 || t_chunk > p->max_t) return fail(CC3D_ESHAPE, "t_chunk=%d not in [1, %d]", t_chunk, p->max_t);
    const Slot& s = p->slots[slot];
    if (s.grouped)
        return fail(CC3D_EINVAL, "slot %d belongs to the frame-batched group and holds only the last batch", slot);
    cc3d_status st = check_frames(p, t_chunk, first != 0);
    if (st != CC3D_OK) return st;
    if (c) *c = s.c;
    if (t) *t = (int)s.tc.eval(t_chunk, first != 0);
    if (h) *h = s.h;
    if (w) *w = s.w;
    clear_err();
    return CC3D_OK;
}

cc3d_status cc3d_slot_read(const cc3d_plan* p, int slot, int t_chunk, int first, void* dst, size_t dst_bytes,
                           void* stream)
{
    if (slot == CC3D_SLOT_AUX) return fail(CC3D_EINVAL, "slot %d is the caller's residual argument", slot);
    int c = 0, t = 0, h = 0, w = 0;
    cc3d_status st = cc3d_slot_shape(p, slot, t_chunk, first, &c, &t, &h, &w);
    if (st != CC3D_OK) return st;
    if (!dst) return fail(CC3D_EINVAL, "dst is NULL");
    const size_t bytes = (size_t)c * t * h * w * p->elem;
    if (dst_bytes < bytes) return fail(CC3D_EINVAL, "dst_bytes=%zu < %zu needed", dst_bytes, bytes);
    DeviceGuard g(p->device);
    st = hip_status(hipMemcpyAsync(dst, p->slots[slot].ptr, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream),
                    "slot copy");
    if (st == CC3D_OK) clear_err();
    return st;
}

cc3d_status cc3d_profile_enable(cc3d_plan* p, int enable)
{
    if (!plan_ok(p)) return fail(CC3D_EINVAL, "plan is NULL or destroyed");
    DeviceGuard g(p->device);
    for (auto& part : p->prof) {
        for (auto& e : part.pending) {
            (void)hipEventSynchronize(e.stop);
            p->event_pool.push_back(e.start);
            p->event_pool.push_back(e.stop);
        }
        part.pending.clear();
        part.launches = 0;
        part.ms = part.flops = part.bytes = 0.0;
    }
    p->prof_on = enable != 0;
    clear_err();
    return CC3D_OK;
}

int cc3d_plan_num_ops(const cc3d_plan* p) { return plan_ok(p) ? (int)p->ops.size() : 0; }

cc3d_status cc3d_profile_read(const cc3d_plan* p, int op, int part, cc3d_op_profile* out)
{
    if (!plan_ok(p)) return fail(CC3D_EINVAL, "plan is NULL or destroyed");
    if (op < 0 || op >= (int)p->ops.size()) return fail(CC3D_EINVAL, "op %d not in [0, %zu)", op, p->ops.size());
    if (part < 0 || part > 2) return fail(CC3D_EINVAL, "part %d not in [0, 2]", part);
    if (!out) return fail(CC3D_EINVAL, "out is NULL");
    DeviceGuard g(p->device);
    auto& pp = p->prof[(size_t)op * 3 + part];
    for (auto& e : pp.pending) {
        hipError_t err = hipEventSynchronize(e.stop);
        float ms = 0.f;
        if (err == hipSuccess) err = hipEventElapsedTime(&ms, e.start, e.stop);
        if (err != hipSuccess) return hip_status(err, "profile event");
        pp.launches += 1;
        pp.ms += ms;
        pp.flops += e.flops;
        pp.bytes += e.bytes;
        p->event_pool.push_back(e.start);
        p->event_pool.push_back(e.stop);
    }
    pp.pending.clear();
    memset(out, 0, sizeof *out);
    snprintf(out->kernel, sizeof out->kernel, "%s", pp.kernel.c_str());
    out->launches = pp.launches;
    out->total_ms = pp.ms;
    out->flops = pp.flops;
    out->bytes = pp.bytes;
    clear_err();
    return CC3D_OK;
}

cc3d_status cc3d_to_channels_last(const void* src, void* dst, int c, int t, int h, int w, int eb, void* stream)
{
    if (!src || !dst) return fail(CC3D_EINVAL, "src or dst is NULL");
    if (c < 1 || t < 1 || h < 1 || w < 1) return fail(CC3D_ESHAPE, "c=%d t=%d h=%d w=%d must be >= 1", c, t, h, w);
    if (eb != 2 && eb != 4) return fail(CC3D_EDTYPE, "elem_bytes=%d; accepted 2 or 4", eb);
    cc3d_status st = hip_status(cc3d::launch_transpose(src, dst, c, (int64_t)t * h * w, eb, (hipStream_t)stream),
                                "transpose launch");
    if (st == CC3D_OK) clear_err();
    return st;
}

cc3d_status cc3d_to_channels_first(const void* src, void* dst, int c, int t, int h, int w, int eb, void* stream)
{
    if (!src || !dst) return fail(CC3D_EINVAL, "src or dst is NULL");
    if (c < 1 || t < 1 || h < 1 || w < 1) return fail(CC3D_ESHAPE, "c=%d t=%d h=%d w=%d must be >= 1", c, t, h, w);
    if (eb != 2 && eb != 4) return fail(CC3D_EDTYPE, "elem_bytes=%d; accepted 2 or 4", eb);
    cc3d_status st = hip_status(cc3d::launch_transpose(src, dst, (int64_t)t * h * w, c, eb, (hipStream_t)stream),
                                "transpose launch");
    if (st == CC3D_OK) clear_err();
    return st;
}

}  // extern "C"

namespace {

cc3d_status forward_impl(const cc3d_plan* p, const void* x, int t_chunk, const cc3d_state* cache_in,
                         cc3d_state* cache_out, const void* residual, void* y, void* stream, bool check_only)
{
    if (!plan_ok(p)) return fail(CC3D_EINVAL, "plan is NULL or destroyed");
    if (!x) return fail(CC3D_EINVAL, "x is NULL");
    if (!y) return fail(CC3D_EINVAL, "y is NULL");
    if (t_chunk < 1 || t_chunk > p->max_t)
        return fail(CC3D_ESHAPE, "t_chunk=%d not in [1, %d] (the plan's max_chunk_t)", t_chunk, p->max_t);
    if (!cache_in || !cache_out) return fail(CC3D_EINVAL, "cache_in or cache_out is NULL");
    if (!cache_in->arena || !cache_out->arena) return fail(CC3D_EINVAL, "a state arena is NULL");
    if (cache_in->arena == cache_out->arena || cache_in == cache_out)
        return fail(CC3D_ESTATE, "cache_in and cache_out share the arena %p; pass two arenas and alternate them",
                    cache_in->arena);
    if (cache_in->frames_seen < 0)
        return fail(CC3D_ESTATE, "cache_in->frames_seen=%lld is negative", (long long)cache_in->frames_seen);
    if (p->uses_aux && !residual) return fail(CC3D_EINVAL, "this plan adds a residual but residual is NULL");
    if (!p->uses_aux && residual) return fail(CC3D_EINVAL, "this plan takes no residual; pass NULL");
    const char* cin_b = (const char*)cache_in->arena;
    const char* cout_b = (const char*)cache_out->arena;
    if (cin_b < cout_b + p->state_bytes && cout_b < cin_b + p->state_bytes)
        return fail(CC3D_ESTATE, "cache_in and cache_out arenas overlap");
    if (((uintptr_t)x | (uintptr_t)y | (uintptr_t)residual | (uintptr_t)cache_in->arena |
         (uintptr_t)cache_out->arena) & 15u)
        return fail(CC3D_EINVAL, "x, y, residual and the state arenas must be 16-byte aligned");
    const bool first = cache_in->frames_seen == 0;
    cc3d_status fst = check_frames(p, t_chunk, first);
    if (fst != CC3D_OK) return fst;
    const Slot& ys = p->slots[CC3D_SLOT_Y];
    const size_t y_bytes = (size_t)ys.tc.eval(t_chunk, first) * ys.h * ys.w * ys.c * p->y_elem;
    const size_t x_bytes = (size_t)t_chunk * p->h * p->w * p->cin * p->elem;
    if ((const char*)x < (const char*)y + y_bytes && (const char*)y < (const char*)x + x_bytes)
        return fail(CC3D_EINVAL, "x and y overlap");

    DeviceGuard g(p->device);
    if (!g.ok) return fail(CC3D_EDEVICE, "cannot make device %d current", p->device);
    cc3d_status st;
    if ((st = check_ptr(x, p->device, "x")) != CC3D_OK) return st;
    if ((st = check_ptr(y, p->device, "y")) != CC3D_OK) return st;
    if ((st = check_ptr(cache_in->arena, p->device, "cache_in arena")) != CC3D_OK) return st;
    if ((st = check_ptr(cache_out->arena, p->device, "cache_out arena")) != CC3D_OK) return st;
    if (residual && (st = check_ptr(residual, p->device, "residual")) != CC3D_OK) return st;
    if (check_only) {
        clear_err();
        return CC3D_OK;
    }

    hipStream_t s = (hipStream_t)stream;
    // One pass of ops over `t` frames of their base input: the chunk input (the
    // whole chunk), or one batch of the frame-batched group's input.
    struct Pass {
        int t;               // frames of the base input
        bool first;          // these are the video's first frames
        const char* cache_rd;  // arena the convs read their history from ...
        char* cache_wr;        // ... and the one their cache updates write
        bool group;          // frame counts relative to the group input
        int64_t in_off;      // group: frame offset into the slots it reads from before the group
        int64_t y_off;       // group: frame offset into y
    };
    auto frames_of = [&](int slot, const Pass& ps) -> int {
        const Slot& sl = p->slots[slot];
        return (int)(ps.group ? sl.rel.eval(ps.t, ps.first) : sl.tc.eval(ps.t, ps.first));
    };
    auto slot_ptr = [&](int slot, const Pass& ps) -> void* {
        if (slot < 0) return nullptr;
        const Slot& sl = p->slots[slot];
        if (slot == CC3D_SLOT_Y)
            return (char*)y + ps.y_off * ((int64_t)sl.h * sl.w * sl.c * p->y_elem);
        char* base = slot == CC3D_SLOT_X ? (char*)const_cast<void*>(x)
                   : slot == CC3D_SLOT_AUX ? (char*)const_cast<void*>(residual) : (char*)sl.ptr;
        if (ps.group && !sl.grouped) base += ps.in_off * ((int64_t)sl.h * sl.w * sl.c * p->elem);
        return base;
    };
    // Caches written by the op that produces the conv's input (pair_cache_writers)
    // in this pass: that conv skips its copy.
    bool cache_written[CC3D_MAX_OPS] = {};
    // Where op r stores the cache of its paired conv for an output of t_s frames
    // (null when the pass has fewer than that conv's kt-1 frames), and the first
    // output frame that goes there.
    auto cache_dest = [&](const OpRt& r, const Pass& ps, int64_t t_s, int64_t* t0) -> void* {
        if (r.cache_to < 0 || ps.group) return nullptr;
        const OpRt& c = p->ops[r.cache_to];
        if (t_s < c.kt - 1) return nullptr;
        *t0 = t_s - (c.kt - 1);
        cache_written[r.cache_to] = true;
        return ps.cache_wr + c.cache_off;
    };
    // rot0: frames of this op's output produced by earlier batches of the chunk
    // (the kernels' temporal-tap rotation follows the frame's place in the chunk,
    // so a batched run sums in the same order as a whole-chunk one)
    auto run_op = [&](const OpRt& r, const Pass& ps, int64_t rot0, int64_t* frames_out) -> cc3d_status {
        cc3d_status st;
        const int t_in = frames_of(r.src, ps);
        const bool first = ps.first;
        if (r.kind == CC3D_OP_CONV) {
            cc3d::ConvArgs a;
            memset(&a, 0, sizeof a);
            a.z.x = slot_ptr(r.src, ps);
            a.z.cache = ps.cache_rd + r.cache_off;
            a.z.frame_elems = (int64_t)r.h_in * r.w_in * r.cin;
            a.z.kt = r.kt;
            a.z.up_t = r.up_t;
            a.z.first = first ? 1 : 0;
            a.z.zero_hist = r.tpad == CC3D_TPAD_ZERO ? 1 : 0;
            a.z.t_shift = (first && !p->grow_aligned) ? 1 : 0;
            // frames of the window's input V, and of the output
            const int t_zv = (r.up_t == 2) ? 2 * t_in - a.z.t_shift : t_in;
            int t_v = t_zv;
            a.down_s = r.stride_s;
            a.t_stride = r.stride_t;
            a.t_first = 0;
            if (r.stride_t == 2) {
                // outputs at input frames tau = phase (mod 2): the chunk's first one
                // is its first frame only on the first chunk with phase 0 (whole
                // counts: later chunks start at an odd frame for phase 0, an even
                // one for phase 1)
                a.t_first = (first && !p->grow_aligned) ? 0 : 1;
                t_v = (t_zv - a.t_first + 1) / 2;
            }
            *frames_out = t_v;
            a.wpk = r.wpk;
            a.bias = r.bias;
            a.res = slot_ptr(r.res, ps);
            a.gamma = r.gamma;
            a.eps = p->eps;
            a.cin = r.cin;
            a.cout = r.cout;
            a.kt = r.kt;
            a.kh = r.kh;
            a.kw = r.kw;
            a.h_in = r.h_in;
            a.w_in = r.w_in;
            a.up_s = r.up_s;
            a.h_out = r.h_out;
            a.w_out = r.w_out;
            a.t_out = t_v;
            a.kchunks = r.kchunks;
            a.ntile = r.ntile;
            a.nblocks = r.nblocks;
            a.family = r.family;
            a.rot_taps = 1;
            a.t_rot0 = (int)rot0;
            a.out_u8 = r.out_u8 ? 1 : 0;
            if (r.fused_act) {
                a.out = slot_ptr(r.out, ps);
                a.act_out = slot_ptr(r.act_out, ps);
            } else {
                a.out = r.act_out != CC3D_SLOT_NONE ? slot_ptr(r.norm_src, ps) : slot_ptr(r.out, ps);
                a.act_out = nullptr;
            }
            const size_t oi = (size_t)(&r - p->ops.data());
            const double vox = (double)t_v * r.h_out * r.w_out;
            const double fr_in = (double)r.h_in * r.w_in * r.cin * p->elem;
            const double fr_out = (double)r.h_out * r.w_out * r.cout * p->elem;
            int64_t c_t0 = 0;
            void* cdst = cache_dest(r, ps, t_v, &c_t0);
            if (cdst && !r.cache_norm) {
                a.cache = cdst;
                a.cache_t0 = (int)c_t0;
                a.cache_act = r.cache_act ? 1 : 0;
            }
            hipError_t e;
            {
                const int nstore = (a.out ? 1 : 0) + (a.act_out ? 1 : 0);
                const double store_scale = r.out_u8 ? 1.0 / p->elem : 1.0;  // 8-bit codes
                const double by = fr_in * (t_in + (first ? 0 : r.kt - 1)) +
                                  (double)r.cout * r.cin * r.kt * r.kh * r.kw * p->elem +
                                  t_v * fr_out * (nstore * store_scale + (a.res ? 1 : 0)) +
                                  (a.cache ? (t_v - c_t0) * fr_out : 0.0);
                ProfScope prof(p, oi, 0, s, 2.0 * r.cin * r.cout * r.kt * r.kh * r.kw * vox, by);
                e = p->dtype == CC3D_BF16 ? cc3d::launch_conv_bf16(a, s) : cc3d::launch_conv_f32(a, s);
            }
            if ((st = hip_status(e, "conv launch")) != CC3D_OK) return st;
            if (r.act_out != CC3D_SLOT_NONE && !r.fused_act) {
                cc3d::NormArgs n;
                memset(&n, 0, sizeof n);
                n.src = slot_ptr(r.norm_src, ps);
                n.act_out = slot_ptr(r.act_out, ps);
                n.gamma = r.gamma;
                n.eps = p->eps;
                n.n_pix = (int64_t)t_v * r.h_out * r.w_out;
                n.c = r.cout;
                if (cdst && r.cache_norm) {
                    n.cache = cdst;
                    n.cache_pix0 = c_t0 * r.h_out * r.w_out;
                    n.cache_act = r.cache_act ? 1 : 0;
                }
                {
                    ProfScope prof(p, oi, 1, s, 0.0, (2.0 * t_v + (n.cache ? t_v - c_t0 : 0)) * fr_out);
                    e = cc3d::launch_norm_act(n, p->elem, s);
                }
                if ((st = hip_status(e, "norm launch")) != CC3D_OK) return st;
            }
            if (r.kt > 1 && !cache_written[oi]) {
                {
                    ProfScope prof(p, oi, 2, s, 0.0, 2.0 * (r.kt - 1) * fr_in);
                    e = cc3d::launch_cache_update(a.z, t_zv, ps.cache_wr + r.cache_off, p->elem, s);
                }
                if ((st = hip_status(e, "cache update launch")) != CC3D_OK) return st;
            }
        } else {
            cc3d::NormArgs n;
            memset(&n, 0, sizeof n);
            n.src = slot_ptr(r.src, ps);
            n.res = slot_ptr(r.res, ps);
            n.out = slot_ptr(r.out, ps);
            n.act_out = slot_ptr(r.act_out, ps);
            n.gamma = r.gamma;
            n.eps = p->eps;
            n.n_pix = (int64_t)t_in * r.h_in * r.w_in;
            n.c = r.cin;
            *frames_out = t_in;
            int64_t c_t0 = 0;
            if ((n.cache = cache_dest(r, ps, t_in, &c_t0)) != nullptr) {
                n.cache_pix0 = c_t0 * r.h_in * r.w_in;
                n.cache_act = r.cache_act ? 1 : 0;
            }
            const size_t oi = (size_t)(&r - p->ops.data());
            const int nmove = 1 + (n.res ? 1 : 0) + (n.out ? 1 : 0) + (n.act_out ? 1 : 0);
            hipError_t e;
            {
                ProfScope prof(p, oi, 0, s, 0.0,
                               (double)n.c * p->elem * (n.n_pix * nmove + (n.cache ? n.n_pix - n.cache_pix0 : 0)));
                e = cc3d::launch_norm_act(n, p->elem, s);
            }
            if ((st = hip_status(e, "norm launch")) != CC3D_OK) return st;
        }
        return CC3D_OK;
    };

    const int n_ops = (int)p->ops.size();
    const int g0 = p->frame_batch > 0 ? p->batch_from : n_ops;
    const Pass whole{t_chunk, first, cin_b, (char*)cache_out->arena, false, 0, 0};
    for (int i = 0; i < g0; ++i) {
        int64_t nf = 0;
        if ((st = run_op(p->ops[i], whole, 0, &nf)) != CC3D_OK) return st;
    }
    if (g0 < n_ops) {
        // The group in batches.  The first batch reads the caches from cache_in,
        // later ones continue the caches the previous batch left in cache_out
        // (the cache update is safe in place).
        const int64_t tg = p->g_in.eval(t_chunk, first);
        std::vector<int64_t> done(n_ops, 0);
        int64_t y_done = 0;
        for (int64_t f0 = 0; f0 < tg; f0 += p->frame_batch) {
            const int tb = (int)std::min<int64_t>(p->frame_batch, tg - f0);
            const bool bfirst = first && f0 == 0;
            const Pass ps{tb, bfirst, f0 == 0 ? cin_b : cout_b, (char*)cache_out->arena, true, f0, y_done};
            for (int i = g0; i < n_ops; ++i) {
                int64_t nf = 0;
                if ((st = run_op(p->ops[i], ps, done[i], &nf)) != CC3D_OK) return st;
                done[i] += nf;
            }
            y_done += p->slots[CC3D_SLOT_Y].rel.eval(tb, bfirst);
        }
    }
    cache_out->frames_seen = cache_in->frames_seen + t_chunk;
    clear_err();
    return CC3D_OK;
}

}  // namespace
