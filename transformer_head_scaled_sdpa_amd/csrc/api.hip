// C ABI of the attention library (declared in include/mha.h).
//
// Every entry point validates all arguments on the host before it enqueues
// anything; kernels run on the caller's stream.  The library allocates no
// device memory: mha_forward's intermediates live in the caller's workspace.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "../../include/mha.h"
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kHeadDim = 64;   // d_k = d_v = d_model / h (the pages' 512 / 8)

size_t elem_size(mha_dtype dt) { return dt == MHA_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == MHA_F32 || dt == MHA_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Byte range [lo, hi) touched by a [B, h, L, d] view with the given strides.
struct Range {
    uintptr_t lo, hi;
};

Range view_range(const void* p, mha_strides s, int B, int h, int L, int d, size_t es) {
    const uintptr_t base = reinterpret_cast<uintptr_t>(p);
    const long long last = (long long)(B - 1) * s.b + (long long)(h - 1) * s.h + (long long)(L - 1) * s.l + d;
    return Range{base, base + (uintptr_t)last * es};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// The bf16 MFMA backward and inspection kernels address one (batch, head)'s
// rows through a buffer resource with 31-bit byte offsets.
bool rows_fit_buffer(long long row_stride, int L, size_t elem) {
    return L <= 0 || (long long)(L - 1) * row_stride * (long long)elem + kHeadDim * (long long)elem < (1ll << 31);
}

// The split-head kernels add 32-bit per-lane byte offsets of up to 128 rows
// to a tile's base address.
bool tile_rows_fit(long long row_stride, size_t elem) { return row_stride * 128 * (long long)elem < (1ll << 31); }

// The multi-head kernels index the [rows, d_model] activations with 32-bit
// element offsets inside a tile and compute row indices as int: each operand
// must hold fewer than 2^31 elements.
bool mha_rows_fit(int B, int L, int d_model) { return (long long)B * L * d_model < (1ll << 31); }

// ---------------------------------------------------------------------------
// kernel timing (a profiling instrument, off unless the calling thread turns
// it on): a pool of HIP event pairs recorded around launches.  The state is
// per thread and created only by mha_timing_enable, so with timing off an
// entry point reads one null thread-local pointer and keeps no state, and
// threads never share a pool.
// ---------------------------------------------------------------------------
constexpr int kPool = 4096;
struct TimingState {
    bool on = false;
    int repeat = 1;      // launches of the kernel inside one event pair
    int used = 0;
    hipEvent_t ev[2 * kPool];
    const char* name[kPool];
};
thread_local TimingState* t_timing = nullptr;

template <typename F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
    TimingState* t = t_timing;
    if (!t || !t->on || t->used >= kPool) return launch();
    const int k = t->used++;
    t->name[k] = name;
    hipError_t e = hipEventRecord(t->ev[2 * k], s);
    if (e != hipSuccess) return e;
    // Every kernel here is a pure function of its inputs, so repeating it
    // leaves the result unchanged; the pair then times `repeat` back-to-back
    // launches and the per-launch average excludes the events' own gaps.
    for (int r = 0; r < t->repeat; ++r) {
        e = launch();
        if (e != hipSuccess) return e;
    }
    return hipEventRecord(t->ev[2 * k + 1], s);
}

mha_status hip_status(hipError_t e) { return e == hipSuccess ? MHA_OK : MHA_EHIP; }

}  // namespace

extern "C" {

const char* mha_status_string(mha_status s) {
    switch (s) {
        case MHA_OK: return "MHA_OK: success";
        case MHA_EINVAL: return "MHA_EINVAL: invalid argument";
        case MHA_ENOTSUP: return "MHA_ENOTSUP: unsupported head width or dtype combination";
        case MHA_EWORKSPACE: return "MHA_EWORKSPACE: workspace too small";
        case MHA_EHIP: return "MHA_EHIP: HIP runtime error while enqueuing";
    }
    return "unknown mha_status";
}

}  // extern "C"

namespace {

// sdpa_backward and sdpa_backward_lse (lse: the forward's log-sum-exp of
// each query, or null).
mha_status backward_impl(mha_dtype in_dt, mha_dtype out_dt,
                         const void* q, mha_strides sq,
                         const void* k, mha_strides sk,
                         const void* v, mha_strides sv,
                         const void* o, mha_strides so,
                         const void* dout, mha_strides sdo,
                         void* dq, mha_strides sdq,
                         void* dk, mha_strides sdk,
                         void* dv, mha_strides sdv,
                         int B, int h, int Lq, int Lk, int d_k, int d_v,
                         const int* valid_lens, int vl_rank, int causal, const float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return MHA_EINVAL;
    if (valid_lens && vl_rank != 1 && vl_rank != 2) return MHA_EINVAL;
    if (B < 0 || h <= 0 || Lq < 0 || Lk <= 0 || d_k <= 0 || d_v <= 0) return MHA_EINVAL;
    if (causal && Lq != Lk) return MHA_EINVAL;
    if (d_k != kHeadDim || d_v != kHeadDim) return MHA_ENOTSUP;
    if (in_dt == MHA_F32 && out_dt != MHA_F32) return MHA_ENOTSUP;
    if (B == 0) return MHA_OK;
    const long long mult = in_dt == MHA_F32 ? 4 : 8, omult = out_dt == MHA_F32 ? 4 : 8;
    const size_t ie = elem_size(in_dt), oe = elem_size(out_dt);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (Lq == 0) {
        // No query rows: dk and dv are sums over nothing, written as zeros.
        if (!dk || !dv || !aligned16(dk) || !aligned16(dv)) return MHA_EINVAL;
        for (const mha_strides& st : {sdk, sdv})
            if (st.b < 0 || st.h < 0 || st.l < 0 || st.b % omult || st.h % omult || st.l % omult) return MHA_EINVAL;
        const Range rk = view_range(dk, sdk, B, h, Lk, d_k, oe), rv = view_range(dv, sdv, B, h, Lk, d_v, oe);
        if (overlap(rk, rv)) return MHA_EINVAL;
        const long long zk[3] = {sdk.b, sdk.h, sdk.l}, zv[3] = {sdv.b, sdv.h, sdv.l};
        hipError_t e = mha::launch_zero_view(dk, zk, B, h, Lk, (int)oe, s);
        if (e == hipSuccess) e = mha::launch_zero_view(dv, zv, B, h, Lk, (int)oe, s);
        return hip_status(e);
    }
    const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return MHA_EINVAL;
    const size_t need = sdpa_backward_workspace_bytes(B, h, Lq);
    if (workspace_bytes < need) return MHA_EWORKSPACE;
    const mha_strides in_s[5] = {sq, sk, sv, so, sdo};
    for (const mha_strides& st : in_s)
        if (st.b < 0 || st.h < 0 || st.l < 0 || st.b % mult || st.h % mult || st.l % mult) return MHA_EINVAL;
    const mha_strides out_s[3] = {sdq, sdk, sdv};
    for (const mha_strides& st : out_s)
        if (st.b < 0 || st.h < 0 || st.l < 0 || st.b % omult || st.h % omult || st.l % omult) return MHA_EINVAL;
    if (in_dt == MHA_BF16 && (!rows_fit_buffer(sq.l, Lq, ie) || !rows_fit_buffer(sdo.l, Lq, ie) ||
                              !rows_fit_buffer(so.l, Lq, ie) || !rows_fit_buffer(sk.l, Lk, ie) ||
                              !rows_fit_buffer(sv.l, Lk, ie) || !tile_rows_fit(sq.l, ie) ||
                              !tile_rows_fit(sdo.l, ie) || !tile_rows_fit(so.l, ie) || !tile_rows_fit(sk.l, ie) ||
                              !tile_rows_fit(sv.l, ie)))
        return MHA_ENOTSUP;
    const uintptr_t wb = reinterpret_cast<uintptr_t>(workspace);
    const Range ins[] = {view_range(q, sq, B, h, Lq, d_k, ie), view_range(k, sk, B, h, Lk, d_k, ie),
                         view_range(v, sv, B, h, Lk, d_v, ie), view_range(o, so, B, h, Lq, d_v, ie),
                         view_range(dout, sdo, B, h, Lq, d_v, ie)};
    const Range outs[] = {view_range(dq, sdq, B, h, Lq, d_k, oe), view_range(dk, sdk, B, h, Lk, d_k, oe),
                          view_range(dv, sdv, B, h, Lk, d_v, oe), Range{wb, wb + need}};
    for (int x = 0; x < 4; ++x) {
        for (const Range& r : ins)
            if (overlap(outs[x], r)) return MHA_EINVAL;
        for (int y = x + 1; y < 4; ++y)
            if (overlap(outs[x], outs[y])) return MHA_EINVAL;
    }
    if (lse) {
        if (reinterpret_cast<uintptr_t>(lse) & 3u) return MHA_EINVAL;
        const uintptr_t lb = reinterpret_cast<uintptr_t>(lse);
        const Range rl{lb, lb + (uintptr_t)B * h * Lq * 4};
        for (const Range& r : outs)
            if (overlap(rl, r)) return MHA_EINVAL;
        if ((long long)B * h * Lq >= (1ll << 31)) return MHA_ENOTSUP;   // query rows index in 32 bits
    }

    mha::BackwardArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout;
    a.dq = dq; a.dk = dk; a.dv = dv;
    const mha_strides* all[8] = {&sq, &sk, &sv, &so, &sdo, &sdq, &sdk, &sdv};
    long long* dst[8] = {a.sq, a.sk, a.sv, a.so, a.sdo, a.sdq, a.sdk, a.sdv};
    for (int x = 0; x < 8; ++x) {
        dst[x][0] = all[x]->b;
        dst[x][1] = all[x]->h;
        dst[x][2] = all[x]->l;
    }
    a.B = B; a.H = h; a.Lq = Lq; a.Lk = Lk;
    a.valid_lens = valid_lens;
    a.vl_rank = valid_lens ? vl_rank : 0;
    a.causal = causal ? 1 : 0;
    a.in_f32 = in_dt == MHA_F32;
    a.out_f32 = out_dt == MHA_F32;
    a.rows = static_cast<float*>(workspace);
    a.lse_in = in_dt == MHA_BF16 ? lse : nullptr;   // the fp32 kernels form their own statistics
    return hip_status(timed("sdpa_backward", s, [&] { return mha::launch_sdpa_backward(a, s); }));
}


// sdpa_forward and sdpa_forward_ex: lengths per sequence (vl_rank 1) or per
// query (2), optional weights p_attn.
mha_status sdpa_impl(mha_dtype in_dt, mha_dtype out_dt,
                     const void* q, mha_strides sq,
                     const void* k, mha_strides sk,
                     const void* v, mha_strides sv,
                     void* o, mha_strides so,
                     int B, int h, int Lq, int Lk, int d_k, int d_v,
                     const int* valid_lens, int vl_rank, int causal,
                     float* p_attn, mha_strides sp, float* lse, void* stream) {
    if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return MHA_EINVAL;
    if (valid_lens && vl_rank != 1 && vl_rank != 2) return MHA_EINVAL;
    if (B < 0 || h <= 0 || Lq < 0 || Lk <= 0 || d_k <= 0 || d_v <= 0) return MHA_EINVAL;
    if (causal && Lq != Lk) return MHA_EINVAL;
    if (d_k != kHeadDim || d_v != kHeadDim) return MHA_ENOTSUP;
    if (in_dt == MHA_F32 && out_dt != MHA_F32) return MHA_ENOTSUP;
    if (B == 0 || Lq == 0) return MHA_OK;
    if (!q || !k || !v || !o) return MHA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return MHA_EINVAL;
    const long long mult = in_dt == MHA_F32 ? 4 : 8;
    const long long omult = out_dt == MHA_F32 ? 4 : 8;
    const mha_strides in_s[3] = {sq, sk, sv};
    for (const mha_strides& s : in_s)
        if (s.b < 0 || s.h < 0 || s.l < 0 || s.b % mult || s.h % mult || s.l % mult) return MHA_EINVAL;
    if (so.b < 0 || so.h < 0 || so.l < 0 || so.b % omult || so.h % omult || so.l % omult) return MHA_EINVAL;
    const size_t ie = elem_size(in_dt), oe = elem_size(out_dt);
    if (!tile_rows_fit(sq.l, ie) || !tile_rows_fit(sk.l, ie) || !tile_rows_fit(sv.l, ie) || !tile_rows_fit(so.l, oe))
        return MHA_ENOTSUP;
    const Range ro = view_range(o, so, B, h, Lq, d_v, oe);
    const Range rq = view_range(q, sq, B, h, Lq, d_k, ie), rk = view_range(k, sk, B, h, Lk, d_k, ie),
                rv = view_range(v, sv, B, h, Lk, d_v, ie);
    if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv)) return MHA_EINVAL;
    if (lse) {
        if (reinterpret_cast<uintptr_t>(lse) & 3u) return MHA_EINVAL;
        const uintptr_t lb = reinterpret_cast<uintptr_t>(lse);
        const Range rl{lb, lb + (uintptr_t)B * h * Lq * 4};
        if (overlap(rl, ro) || overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv)) return MHA_EINVAL;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p_attn || (valid_lens && vl_rank == 2)) {
        if (in_dt == MHA_BF16 && (!rows_fit_buffer(sk.l, Lk, ie) || !rows_fit_buffer(sv.l, Lk, ie))) return MHA_ENOTSUP;
        if (p_attn) {
            if (reinterpret_cast<uintptr_t>(p_attn) & 3u) return MHA_EINVAL;
            if (sp.b < 0 || sp.h < 0 || sp.l < 0) return MHA_EINVAL;
            const Range rp = view_range(p_attn, sp, B, h, Lq, Lk, 4);
            if (overlap(rp, ro) || overlap(rp, rq) || overlap(rp, rk) || overlap(rp, rv)) return MHA_EINVAL;
        }
        mha::WeightsArgs w;
        w.q = q; w.k = k; w.v = v; w.o = o;
        w.sq[0] = sq.b; w.sq[1] = sq.h; w.sq[2] = sq.l;
        w.sk[0] = sk.b; w.sk[1] = sk.h; w.sk[2] = sk.l;
        w.sv[0] = sv.b; w.sv[1] = sv.h; w.sv[2] = sv.l;
        w.so[0] = so.b; w.so[1] = so.h; w.so[2] = so.l;
        w.B = B; w.H = h; w.Lq = Lq; w.Lk = Lk;
        w.valid_lens = valid_lens;
        w.vl_rank = valid_lens ? vl_rank : 0;
        w.causal = causal ? 1 : 0;
        w.in_f32 = in_dt == MHA_F32;
        w.out_f32 = out_dt == MHA_F32;
        w.p = p_attn;
        w.sp[0] = sp.b; w.sp[1] = sp.h; w.sp[2] = sp.l;
        return hip_status(timed("sdpa_weights", s, [&] { return mha::launch_sdpa_weights(w, s); }));
    }

    mha::SdpaArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.sq[0] = sq.b; a.sq[1] = sq.h; a.sq[2] = sq.l;
    a.sk[0] = sk.b; a.sk[1] = sk.h; a.sk[2] = sk.l;
    a.sv[0] = sv.b; a.sv[1] = sv.h; a.sv[2] = sv.l;
    a.so[0] = so.b; a.so[1] = so.h; a.so[2] = so.l;
    a.B = B; a.H = h; a.Lq = Lq; a.Lk = Lk;
    a.valid_lens = valid_lens;
    a.causal = causal ? 1 : 0;
    a.lse = lse;
    if (in_dt == MHA_F32) return hip_status(timed("sdpa_f32", s, [&] { return mha::launch_sdpa_f32(a, s); }));
    return hip_status(timed("sdpa_bf16", s, [&] { return mha::launch_sdpa_bf16(a, out_dt == MHA_F32, s); }));
}

}  // namespace

extern "C" {

mha_status sdpa_forward(mha_dtype in_dt, mha_dtype out_dt,
                        const void* q, mha_strides sq,
                        const void* k, mha_strides sk,
                        const void* v, mha_strides sv,
                        void* o, mha_strides so,
                        int B, int h, int Lq, int Lk, int d_k, int d_v,
                        const int* valid_lens, int causal, void* stream) {
    return sdpa_impl(in_dt, out_dt, q, sq, k, sk, v, sv, o, so, B, h, Lq, Lk, d_k, d_v, valid_lens, 1, causal,
                     nullptr, mha_strides{0, 0, 0}, nullptr, stream);
}

mha_status sdpa_forward_lse(mha_dtype in_dt, mha_dtype out_dt,
                            const void* q, mha_strides sq,
                            const void* k, mha_strides sk,
                            const void* v, mha_strides sv,
                            void* o, mha_strides so,
                            int B, int h, int Lq, int Lk, int d_k, int d_v,
                            const int* valid_lens, int causal, float* lse, void* stream) {
    if (!lse && B > 0 && Lq > 0) return MHA_EINVAL;
    return sdpa_impl(in_dt, out_dt, q, sq, k, sk, v, sv, o, so, B, h, Lq, Lk, d_k, d_v, valid_lens, 1, causal,
                     nullptr, mha_strides{0, 0, 0}, lse, stream);
}

mha_status sdpa_forward_ex(mha_dtype in_dt, mha_dtype out_dt,
                           const void* q, mha_strides sq,
                           const void* k, mha_strides sk,
                           const void* v, mha_strides sv,
                           void* o, mha_strides so,
                           int B, int h, int Lq, int Lk, int d_k, int d_v,
                           const int* valid_lens, int vl_rank, int causal,
                           float* p_attn, mha_strides sp, void* stream) {
    return sdpa_impl(in_dt, out_dt, q, sq, k, sk, v, sv, o, so, B, h, Lq, Lk, d_k, d_v, valid_lens, vl_rank,
                     causal, p_attn, sp, nullptr, stream);
}

size_t sdpa_backward_workspace_bytes(int B, int h, int Lq) {
    if (B < 0 || h <= 0 || Lq < 0) return 0;
    return round_up(mha::backward_workspace_bytes(B, h, Lq), 256);
}

mha_status sdpa_backward(mha_dtype in_dt, mha_dtype out_dt,
                         const void* q, mha_strides sq,
                         const void* k, mha_strides sk,
                         const void* v, mha_strides sv,
                         const void* o, mha_strides so,
                         const void* dout, mha_strides sdo,
                         void* dq, mha_strides sdq,
                         void* dk, mha_strides sdk,
                         void* dv, mha_strides sdv,
                         int B, int h, int Lq, int Lk, int d_k, int d_v,
                         const int* valid_lens, int vl_rank, int causal,
                         void* workspace, size_t workspace_bytes, void* stream) {
    return backward_impl(in_dt, out_dt, q, sq, k, sk, v, sv, o, so, dout, sdo, dq, sdq, dk, sdk, dv, sdv, B, h, Lq,
                         Lk, d_k, d_v, valid_lens, vl_rank, causal, nullptr, workspace, workspace_bytes, stream);
}

mha_status sdpa_backward_lse(mha_dtype in_dt, mha_dtype out_dt,
                             const void* q, mha_strides sq,
                             const void* k, mha_strides sk,
                             const void* v, mha_strides sv,
                             const void* o, mha_strides so,
                             const void* dout, mha_strides sdo,
                             void* dq, mha_strides sdq,
                             void* dk, mha_strides sdk,
                             void* dv, mha_strides sdv,
                             int B, int h, int Lq, int Lk, int d_k, int d_v,
                             const int* valid_lens, int vl_rank, int causal, const float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (!lse && B > 0 && Lq > 0) return MHA_EINVAL;
    return backward_impl(in_dt, out_dt, q, sq, k, sk, v, sv, o, so, dout, sdo, dq, sdq, dk, sdk, dv, sdv, B, h, Lq,
                         Lk, d_k, d_v, valid_lens, vl_rank, causal, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------------------
// sdpa_decode and its allocation-free variant
// ---------------------------------------------------------------------------
// The allocation-free variant keeps the per-split partials of a decoding step
// in this file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends; every call on a
// GPU shares it (calls that overlap on one GPU race on it).  No part of it
// has to start at zero: each launch writes every partial it later reads.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current (in host code the array's name is only a stand-in).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

mha_status decode_scratch(void** addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MHA_EHIP;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MHA_EHIP;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *addr = p;
    return MHA_OK;
}

// use_scratch: the partials go to the device's `scratch` array (workspace and
// workspace_bytes are ignored), and steps that need more than it holds are
// refused with MHA_EWORKSPACE.
mha_status decode_impl(mha_dtype in_dt, mha_dtype out_dt,
                       const void* q, mha_strides sq,
                       const void* k, mha_strides sk,
                       const void* v, mha_strides sv,
                       void* o, mha_strides so,
                       int B, int h, int L, int d_k, int d_v, const int* lens,
                       bool use_scratch, void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return MHA_EINVAL;
    if (B < 0 || h <= 0 || L <= 0 || d_k <= 0 || d_v <= 0) return MHA_EINVAL;
    if (d_k != kHeadDim || d_v != kHeadDim || in_dt != MHA_BF16) return MHA_ENOTSUP;
    if (B == 0) return MHA_OK;
    if (!q || !k || !v || !o || !lens || (!use_scratch && !workspace)) return MHA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (!use_scratch && !aligned16(workspace)))
        return MHA_EINVAL;
    const long long omult = out_dt == MHA_F32 ? 4 : 8;
    const mha_strides in_s[3] = {sq, sk, sv};
    for (const mha_strides& s : in_s)
        if (s.b < 0 || s.h < 0 || s.l < 0 || s.b % 8 || s.h % 8 || s.l % 8) return MHA_EINVAL;
    // A slice's 512 cached rows are addressed with 31-bit byte offsets.
    if (sk.l * 2 * 512 >= (1ll << 31) || sv.l * 2 * 512 >= (1ll << 31)) return MHA_ENOTSUP;
    if (so.b < 0 || so.h < 0 || so.b % omult || so.h % omult) return MHA_EINVAL;
    const size_t need = round_up(mha::decode_workspace_bytes(B, h, L), 256);
    if (use_scratch ? need > kDecodeScratchBytes : workspace_bytes < need) return MHA_EWORKSPACE;
    const size_t oe = elem_size(out_dt);
    const mha_strides so1{so.b, so.h, 0};
    const Range ro = view_range(o, so1, B, h, 1, d_v, oe);
    const mha_strides sq1{sq.b, sq.h, 0};
    const Range ins[3] = {view_range(q, sq1, B, h, 1, d_k, 2), view_range(k, sk, B, h, L, d_k, 2),
                          view_range(v, sv, B, h, L, d_v, 2)};
    for (const Range& r : ins)
        if (overlap(ro, r)) return MHA_EINVAL;
    if (!use_scratch) {
        const uintptr_t wb = reinterpret_cast<uintptr_t>(workspace);
        const Range rw{wb, wb + need};
        for (const Range& r : ins)
            if (overlap(rw, r)) return MHA_EINVAL;
        if (overlap(ro, rw)) return MHA_EINVAL;
    } else {
        const mha_status st = decode_scratch(&workspace);
        if (st != MHA_OK) return st;
    }

    mha::DecodeArgs d;
    d.q = q; d.k = k; d.v = v; d.o = o;
    d.sq[0] = sq.b; d.sq[1] = sq.h;
    d.sk[0] = sk.b; d.sk[1] = sk.h; d.sk[2] = sk.l;
    d.sv[0] = sv.b; d.sv[1] = sv.h; d.sv[2] = sv.l;
    d.so[0] = so.b; d.so[1] = so.h;
    d.B = B; d.H = h; d.L = L;
    d.lens = lens;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(timed("sdpa_decode", s, [&] {
        return mha::launch_sdpa_decode(d, out_dt == MHA_F32, workspace, s);
    }));
}

}  // namespace

extern "C" {

size_t sdpa_decode_workspace_bytes(int B, int h, int L) {
    if (B < 0 || h <= 0 || L <= 0) return 0;
    return round_up(mha::decode_workspace_bytes(B, h, L), 256);
}

mha_status sdpa_decode(mha_dtype in_dt, mha_dtype out_dt,
                       const void* q, mha_strides sq,
                       const void* k, mha_strides sk,
                       const void* v, mha_strides sv,
                       void* o, mha_strides so,
                       int B, int h, int L, int d_k, int d_v, const int* lens,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(in_dt, out_dt, q, sq, k, sk, v, sv, o, so, B, h, L, d_k, d_v, lens, false, workspace,
                       workspace_bytes, stream);
}

mha_status sdpa_decode_noalloc(mha_dtype in_dt, mha_dtype out_dt,
                               const void* q, mha_strides sq,
                               const void* k, mha_strides sk,
                               const void* v, mha_strides sv,
                               void* o, mha_strides so,
                               int B, int h, int L, int d_k, int d_v, const int* lens, void* stream) {
    return decode_impl(in_dt, out_dt, q, sq, k, sk, v, sv, o, so, B, h, L, d_k, d_v, lens, true, nullptr, 0,
                       stream);
}

size_t mha_workspace_bytes(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h) {
    if (!valid_dtype(in_dt) || B < 0 || Lq < 0 || Lk < 0 || d_model <= 0 || h <= 0 || d_model % h) return 0;
    const size_t es = elem_size(in_dt);
    const size_t q = round_up((size_t)B * Lq * d_model * es, 256);
    const size_t kv = round_up((size_t)B * Lk * d_model * es, 256);
    // fp32: Q, K, V, merged heads.  bf16: merged heads, Q hi and lo, K hi and
    // lo, V (the projected route; the single-pass route for short
    // self-attention uses only the merged heads, but the shapes alone do not
    // tell self- from cross-attention).
    return in_dt == MHA_BF16 ? 3 * q + 3 * kv : 2 * q + 2 * kv;
}

size_t mha_workspace_bytes_ex(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h) {
    if (!valid_dtype(in_dt) || B < 0 || Lq < 0 || Lk < 0 || d_model <= 0 || h <= 0 || d_model % h) return 0;
    // merged heads in in_dt, then Q, K, V in fp32
    return round_up((size_t)B * Lq * d_model * elem_size(in_dt), 256) + round_up((size_t)B * Lq * d_model * 4, 256) +
           2 * round_up((size_t)B * Lk * d_model * 4, 256);
}

}  // extern "C"

namespace {

// The bf16 multi-head layer projects K and V inside its attention kernel for
// every block of 256 queries, so it repeats that work n = ceil(Lq / 256)
// times without the causal rule and (n + 1) / 2 times with it (block i needs
// keys below (i + 1) * 256).  Measured on MI355X against the projected route
// (one GEMM launch for Q, K, V, then attention on the projections): the
// single kernel is faster or equal up to a factor of 1.5 with at most 512
// keys (B64 L512 causal: 174 against 188 us; B16 Lq256 Lk384: 85 against
// 85 us); beyond that the projected route wins (B4 L1024 causal 85 against
// 52 us; B16 L512 non-causal d_model 1024: 182 against 142 us; B8 Lq256
// Lk768: 66 against 47 us).
bool fused_route_pays(int Lq, int Lk, bool causal) {
    const long long n = (Lq + 255) / 256;
    const long long twice_factor = causal ? n + 1 : 2 * n;   // 2 x re-projection factor
    return twice_factor <= 3 && Lk <= 512;
}

// mha_forward and mha_forward_ex (lengths per query, optional weights).
mha_status mha_impl(mha_dtype in_dt, mha_dtype out_dt,
                    const void* x_q, const void* x_kv,
                    const void* w_q, const void* b_q,
                    const void* w_k, const void* b_k,
                    const void* w_v, const void* b_v,
                    const void* w_o, const void* b_o,
                    void* out,
                    int B, int Lq, int Lk, int d_model, int h, int d_k,
                    const int* valid_lens, int vl_rank, int causal, float* p_attn, mha_strides sp,
                    void* workspace, size_t workspace_bytes, void* stream, const void* residual = nullptr) {
    if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return MHA_EINVAL;
    if (valid_lens && vl_rank != 1 && vl_rank != 2) return MHA_EINVAL;
    // The inspection path: projections to fp32, attention with the weights.
    const bool ex = p_attn || (valid_lens && vl_rank == 2);
    if (B < 0 || Lq < 0 || Lk <= 0 || d_model <= 0 || h <= 0 || d_k <= 0) return MHA_EINVAL;
    if ((long long)h * d_k != d_model) return MHA_EINVAL;
    if (causal && Lq != Lk) return MHA_EINVAL;
    if (d_k != kHeadDim) return MHA_ENOTSUP;
    if (in_dt == MHA_F32 && out_dt != MHA_F32) return MHA_ENOTSUP;
    if (B == 0 || Lq == 0) return MHA_OK;
    if (!mha_rows_fit(B, Lq, d_model) || !mha_rows_fit(B, Lk, d_model)) return MHA_ENOTSUP;
    if (!x_q || !x_kv || !w_q || !w_k || !w_v || !w_o || !out || !workspace) return MHA_EINVAL;
    const void* ptrs[] = {x_q, x_kv, w_q, w_k, w_v, w_o, out, workspace, b_q, b_k, b_v, b_o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MHA_EINVAL;
    const size_t need = ex ? mha_workspace_bytes_ex(in_dt, B, Lq, Lk, d_model, h)
                           : mha_workspace_bytes(in_dt, B, Lq, Lk, d_model, h);
    if (workspace_bytes < need) return MHA_EWORKSPACE;

    const size_t ie = elem_size(in_dt), oe = elem_size(out_dt);
    const uintptr_t ob = reinterpret_cast<uintptr_t>(out);
    const Range rout{ob, ob + (size_t)B * Lq * d_model * oe};
    const uintptr_t wb = reinterpret_cast<uintptr_t>(workspace);
    const Range inputs[] = {
        {reinterpret_cast<uintptr_t>(x_q), reinterpret_cast<uintptr_t>(x_q) + (size_t)B * Lq * d_model * ie},
        {reinterpret_cast<uintptr_t>(x_kv), reinterpret_cast<uintptr_t>(x_kv) + (size_t)B * Lk * d_model * ie},
        {reinterpret_cast<uintptr_t>(w_q), reinterpret_cast<uintptr_t>(w_q) + (size_t)d_model * d_model * ie},
        {reinterpret_cast<uintptr_t>(w_k), reinterpret_cast<uintptr_t>(w_k) + (size_t)d_model * d_model * ie},
        {reinterpret_cast<uintptr_t>(w_v), reinterpret_cast<uintptr_t>(w_v) + (size_t)d_model * d_model * ie},
        {reinterpret_cast<uintptr_t>(w_o), reinterpret_cast<uintptr_t>(w_o) + (size_t)d_model * d_model * ie},
        {wb, wb + need},
    };
    for (const Range& r : inputs)
        if (overlap(rout, r)) return MHA_EINVAL;
    const Range rws{wb, wb + need};
    for (int n = 0; n < 6; ++n)
        if (overlap(rws, inputs[n])) return MHA_EINVAL;
    const void* biases[] = {b_q, b_k, b_v, b_o};
    for (const void* p : biases) {
        if (!p) continue;
        const Range rb{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + (size_t)d_model * ie};
        if (overlap(rout, rb) || overlap(rws, rb)) return MHA_EINVAL;
    }
    if (p_attn) {
        if (reinterpret_cast<uintptr_t>(p_attn) & 3u) return MHA_EINVAL;
        if (sp.b < 0 || sp.h < 0 || sp.l < 0) return MHA_EINVAL;
        const Range rp = view_range(p_attn, sp, B, h, Lq, Lk, 4);
        if (overlap(rp, rout)) return MHA_EINVAL;
        for (const Range& r : inputs)
            if (overlap(rp, r)) return MHA_EINVAL;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(workspace);
    const bool bf16 = in_dt == MHA_BF16;
    void* Ocat = w;
    hipError_t e;
    if (ex) {
        // Workspace: merged heads [B*Lq, D] (in_dt), then fp32 Q [B*Lq, D], K, V [B*Lk, D].
        char* Q = w + round_up((size_t)B * Lq * d_model * ie, 256);
        char* K = Q + round_up((size_t)B * Lq * d_model * 4, 256);
        char* V = K + round_up((size_t)B * Lk * d_model * 4, 256);
        mha::GemmArgs g;
        g.nprob = 3;
        g.N = d_model;
        g.K = d_model;
        g.p[0] = {x_q, w_q, b_q, Q, B * Lq};
        g.p[1] = {x_kv, w_k, b_k, K, B * Lk};
        g.p[2] = {x_kv, w_v, b_v, V, B * Lk};
        e = timed("qkv_proj_ex", s, [&] { return bf16 ? mha::launch_gemm_bf16(g, true, s) : mha::launch_gemm_f32(g, s); });
        if (e != hipSuccess) return MHA_EHIP;
        mha::WeightsArgs a;
        a.q = Q; a.k = K; a.v = V; a.o = Ocat;
        a.sq[0] = (long long)Lq * d_model; a.sq[1] = d_k; a.sq[2] = d_model;
        a.sk[0] = (long long)Lk * d_model; a.sk[1] = d_k; a.sk[2] = d_model;
        a.sv[0] = (long long)Lk * d_model; a.sv[1] = d_k; a.sv[2] = d_model;
        a.so[0] = (long long)Lq * d_model; a.so[1] = d_k; a.so[2] = d_model;
        a.B = B; a.H = h; a.Lq = Lq; a.Lk = Lk;
        a.valid_lens = valid_lens;
        a.vl_rank = valid_lens ? vl_rank : 0;
        a.causal = causal ? 1 : 0;
        a.in_f32 = true;
        a.out_f32 = !bf16;
        a.p = p_attn;
        a.sp[0] = sp.b; a.sp[1] = sp.h; a.sp[2] = sp.l;
        e = timed("sdpa_weights", s, [&] { return mha::launch_sdpa_weights(a, s); });
        if (e != hipSuccess) return MHA_EHIP;
    } else if (bf16) {
        mha::FusedArgs f;
        f.x_q = x_q; f.x_kv = x_kv;
        f.w_q = w_q; f.w_k = w_k; f.w_v = w_v;
        f.b_q = b_q; f.b_k = b_k; f.b_v = b_v;
        f.o = Ocat;
        f.B = B; f.H = h; f.Lq = Lq; f.Lk = Lk; f.D = d_model;
        f.valid_lens = valid_lens;
        f.causal = causal ? 1 : 0;
        if (mha::mha_attn_fused_small_fits(f) || fused_route_pays(Lq, Lk, causal != 0)) {
            // 1-2. Q/K/V projections, head split, attention and head merge in
            // one kernel (K and V projected on chip for each block of
            // queries); the merged heads land in the workspace.
            e = timed("attn_fused_bf16", s, [&] { return mha::launch_mha_attn_fused(f, s); });
            if (e != hipSuccess) return MHA_EHIP;
        } else {
            // 1. Q/K/V projections in one launch (three problems): Q times
            // log2(e)/sqrt(d_k) and K as bf16 hi + lo planes, V in bf16.
            // Workspace: merged heads [B*Lq, D], Q hi, Q lo [B*Lq, D], K hi,
            // K lo, V [B*Lk, D], all bf16.
            const size_t qb = round_up((size_t)B * Lq * d_model * 2, 256);
            const size_t kb = round_up((size_t)B * Lk * d_model * 2, 256);
            char* Qh = w + qb;
            char* Ql = Qh + qb;
            char* Kh = Ql + qb;
            char* Kl = Kh + kb;
            char* V = Kl + kb;
            mha::GemmArgs g;
            g.nprob = 3;
            g.N = d_model;
            g.K = d_model;
            g.p[0] = {x_q, w_q, b_q, Qh, B * Lq};
            g.p[0].c_lo = Ql;
            g.p[0].scale = mha::kLog2e / 8.0f;   // log2(e) / sqrt(64)
            g.p[1] = {x_kv, w_k, b_k, Kh, B * Lk};
            g.p[1].c_lo = Kl;
            g.p[2] = {x_kv, w_v, b_v, V, B * Lk};
            e = timed("qkv_proj_bf16", s, [&] { return mha::launch_gemm_bf16(g, false, s); });
            if (e != hipSuccess) return MHA_EHIP;
            // 2. Attention per head over [B*L, D] viewed as [B, L, h, d_k],
            // scores from the three hi/lo products.
            mha::SdpaArgs a;
            a.q = Qh; a.q_lo = Ql; a.k = Kh; a.k_lo = Kl; a.v = V; a.o = Ocat;
            a.sq[0] = (long long)Lq * d_model; a.sq[1] = d_k; a.sq[2] = d_model;
            a.sk[0] = (long long)Lk * d_model; a.sk[1] = d_k; a.sk[2] = d_model;
            a.sv[0] = (long long)Lk * d_model; a.sv[1] = d_k; a.sv[2] = d_model;
            a.so[0] = (long long)Lq * d_model; a.so[1] = d_k; a.so[2] = d_model;
            a.B = B; a.H = h; a.Lq = Lq; a.Lk = Lk;
            a.valid_lens = valid_lens;
            a.causal = causal ? 1 : 0;
            e = timed("sdpa_hilo_bf16", s, [&] { return mha::launch_sdpa_bf16(a, false, s); });
            if (e != hipSuccess) return MHA_EHIP;
        }
    } else {
        // Workspace: merged heads [B*Lq, D], Q [B*Lq, D], K [B*Lk, D], V [B*Lk, D].
        const size_t qbytes = round_up((size_t)B * Lq * d_model * ie, 256);
        const size_t kvbytes = round_up((size_t)B * Lk * d_model * ie, 256);
        void* Q = w + qbytes;
        void* K = w + 2 * qbytes;
        void* V = w + 2 * qbytes + kvbytes;

        // 1. Q/K/V projections in one launch (three problems).
        mha::GemmArgs g;
        g.nprob = 3;
        g.N = d_model;
        g.K = d_model;
        g.p[0] = {x_q, w_q, b_q, Q, B * Lq};
        g.p[1] = {x_kv, w_k, b_k, K, B * Lk};
        g.p[2] = {x_kv, w_v, b_v, V, B * Lk};
        e = timed("qkv_proj_f32", s, [&] { return mha::launch_gemm_f32(g, s); });
        if (e != hipSuccess) return MHA_EHIP;

        // 2. Attention per head: [B*L, D] row-major viewed as [B, L, h, d_k].
        mha::SdpaArgs a;
        a.q = Q; a.k = K; a.v = V; a.o = Ocat;
            a.sq[0] = (long long)Lq * d_model; a.sq[1] = d_k; a.sq[2] = d_model;
        a.sk[0] = (long long)Lk * d_model; a.sk[1] = d_k; a.sk[2] = d_model;
        a.sv[0] = (long long)Lk * d_model; a.sv[1] = d_k; a.sv[2] = d_model;
        a.so[0] = (long long)Lq * d_model; a.so[1] = d_k; a.so[2] = d_model;
        a.B = B; a.H = h; a.Lq = Lq; a.Lk = Lk;
        a.valid_lens = valid_lens;
        a.causal = causal ? 1 : 0;
        e = timed("sdpa_f32", s, [&] { return mha::launch_sdpa_f32(a, s); });
        if (e != hipSuccess) return MHA_EHIP;
    }

    // 3. Output projection of the merged heads.
    mha::GemmArgs go;
    go.nprob = 1;
    go.N = d_model;
    go.K = d_model;
    go.p[0] = {Ocat, w_o, b_o, out, B * Lq, residual};
    e = timed(bf16 ? "out_proj_bf16" : "out_proj_f32", s, [&] {
        return bf16 ? mha::launch_gemm_bf16(go, out_dt == MHA_F32, s) : mha::launch_gemm_f32(go, s);
    });
    return hip_status(e);
}

}  // namespace

extern "C" {

mha_status mha_forward(mha_dtype in_dt, mha_dtype out_dt,
                       const void* x_q, const void* x_kv,
                       const void* w_q, const void* b_q,
                       const void* w_k, const void* b_k,
                       const void* w_v, const void* b_v,
                       const void* w_o, const void* b_o,
                       void* out,
                       int B, int Lq, int Lk, int d_model, int h, int d_k,
                       const int* valid_lens, int causal,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return mha_impl(in_dt, out_dt, x_q, x_kv, w_q, b_q, w_k, b_k, w_v, b_v, w_o, b_o, out, B, Lq, Lk, d_model, h,
                    d_k, valid_lens, 1, causal, nullptr, mha_strides{0, 0, 0}, workspace, workspace_bytes, stream);
}

mha_status mha_forward_ex(mha_dtype in_dt, mha_dtype out_dt,
                          const void* x_q, const void* x_kv,
                          const void* w_q, const void* b_q,
                          const void* w_k, const void* b_k,
                          const void* w_v, const void* b_v,
                          const void* w_o, const void* b_o,
                          void* out,
                          int B, int Lq, int Lk, int d_model, int h, int d_k,
                          const int* valid_lens, int vl_rank, int causal, float* p_attn, mha_strides sp,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return mha_impl(in_dt, out_dt, x_q, x_kv, w_q, b_q, w_k, b_k, w_v, b_v, w_o, b_o, out, B, Lq, Lk, d_model, h,
                    d_k, valid_lens, vl_rank, causal, p_attn, sp, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Workspace of mha_backward, byte offsets (each 256-byte aligned): Q, K, V,
// the merged heads and their gradient (bf16), the log-sum-exp and the
// attention backward's row statistics (fp32), dQ, dK, dV (bf16: one [M, 3D]
// block for the fused input gradient of self-attention, or dQ [Mq, D] then
// [dK | dV] [Mk, 2D]), the transposed weights (bf16: W_o^T, then W_q^T,
// W_k^T, W_v^T side by side or apart) and the weight-gradient partials.
// With `forward` false the forward's tensors (Q, K, V, merged heads,
// log-sum-exp) are not in the workspace: they come from mha_forward_train's
// saved buffer, whose layout is the same five segments (SavedLayout).
struct BwdLayout {
    size_t q, k, v, ocat, docat, lse, rows, dqkv, dkv, wt, tn, total;
};

struct SavedLayout {
    size_t q, k, v, ocat, lse, total;
};

SavedLayout saved_layout(int B, int Lq, int Lk, int D, int h) {
    SavedLayout L{};
    size_t off = 0;
    auto take = [&](size_t n) {
        const size_t o = off;
        off = round_up(off + n, 256);
        return o;
    };
    const size_t mq = (size_t)B * Lq * D * 2, mk = (size_t)B * Lk * D * 2;
    L.q = take(mq);
    L.k = take(mk);
    L.v = take(mk);
    L.ocat = take(mq);
    L.lse = take((size_t)B * h * Lq * 4);
    L.total = off;
    return L;
}

BwdLayout bwd_layout(int B, int Lq, int Lk, int D, int h, bool forward = true) {
    BwdLayout L{};
    size_t off = 0;
    if (forward) {
        const SavedLayout S = saved_layout(B, Lq, Lk, D, h);
        L.q = S.q;
        L.k = S.k;
        L.v = S.v;
        L.ocat = S.ocat;
        L.lse = S.lse;
        off = S.total;
    }
    auto take = [&](size_t n) {
        const size_t o = off;
        off = round_up(off + n, 256);
        return o;
    };
    const size_t mq = (size_t)B * Lq * D * 2, mk = (size_t)B * Lk * D * 2;
    L.docat = take(mq);
    L.rows = take(mha::backward_workspace_bytes(B, h, Lq));
    L.dqkv = take(round_up(mq, 256) + 2 * mk);
    L.dkv = L.dqkv + round_up(mq, 256);
    L.wt = take((size_t)4 * D * D * 2);
    const int M[3] = {B * Lq, B * Lq, B * Lk}, N1[3] = {D, D, 2 * D}, N2[3] = {D, D, D};
    L.tn = take(mha::gemm_tn_workspace_bytes(M, N1, N2, 3));
    L.total = off;
    return L;
}

// Sizes the multi-head training entry points accept (shared checks).
bool mha_train_sizes_ok(int B, int Lq, int Lk, int d_model, int h) {
    return B >= 0 && Lq >= 0 && Lk >= 0 && d_model > 0 && h > 0 && d_model % h == 0 && d_model % 64 == 0 &&
           mha_rows_fit(B, Lq, 6 * d_model) && mha_rows_fit(B, Lk, 6 * d_model);
}

// mha_backward (saved == nullptr: the forward is recomputed into the
// workspace) and mha_backward_saved (the forward's tensors from `saved`).
mha_status mha_backward_impl(mha_dtype in_dt,
                             const void* x_q, const void* x_kv,
                             const void* w_q, const void* b_q,
                             const void* w_k, const void* b_k,
                             const void* w_v, const void* b_v,
                             const void* w_o,
                             const void* saved, size_t saved_bytes,
                             const void* dout,
                             float* dx_q, float* dx_kv,
                             float* dw_q, float* db_q,
                             float* dw_k, float* db_k,
                             float* dw_v, float* db_v,
                             float* dw_o, float* db_o,
                             int B, int Lq, int Lk, int d_model, int h, int d_k,
                             const int* valid_lens, int causal,
                             void* workspace, size_t workspace_bytes, void* stream, bool use_saved) {
    if (!valid_dtype(in_dt)) return MHA_EINVAL;
    if (B < 0 || Lq < 0 || Lk <= 0 || d_model <= 0 || h <= 0 || d_k <= 0) return MHA_EINVAL;
    if ((long long)h * d_k != d_model) return MHA_EINVAL;
    if (causal && Lq != Lk) return MHA_EINVAL;
    if (d_k != kHeadDim || in_dt != MHA_BF16) return MHA_ENOTSUP;
    const int D = d_model;
    const bool any_db = db_q || db_k || db_v || db_o, all_db = db_q && db_k && db_v && db_o;
    if (any_db && !all_db) return MHA_EINVAL;
    if (!dw_q || !dw_k || !dw_v || !dw_o) return MHA_EINVAL;
    // dx_kv == NULL: self-attention, dx_q takes both paths.
    const bool fused_dx = dx_kv == nullptr;
    if (fused_dx && (x_kv != x_q || Lq != Lk)) return MHA_EINVAL;
    if (!mha_rows_fit(B, Lq, 6 * D) || !mha_rows_fit(B, Lk, 6 * D)) return MHA_ENOTSUP;

    // Output ranges (fp32).
    const size_t dd = (size_t)D * D * 4;
    auto rng = [](const void* p, size_t n) {
        const uintptr_t b = reinterpret_cast<uintptr_t>(p);
        return Range{b, b + n};
    };
    Range outs[10];
    int n_out = 0;
    for (float* p : {dw_q, dw_k, dw_v, dw_o}) {
        if (!aligned16(p)) return MHA_EINVAL;
        outs[n_out++] = rng(p, dd);
    }
    if (all_db)
        for (float* p : {db_q, db_k, db_v, db_o}) {
            if (reinterpret_cast<uintptr_t>(p) & 3u) return MHA_EINVAL;
            outs[n_out++] = rng(p, (size_t)D * 4);
        }
    if (dx_kv) {
        if (!aligned16(dx_kv)) return MHA_EINVAL;
        outs[n_out++] = rng(dx_kv, (size_t)B * Lk * D * 4);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool empty = B == 0 || Lq == 0;
    if (!empty) {
        if (!dx_q || !aligned16(dx_q)) return MHA_EINVAL;
        outs[n_out++] = rng(dx_q, (size_t)B * Lq * D * 4);
    }
    for (int x = 0; x < n_out; ++x)
        for (int y = x + 1; y < n_out; ++y)
            if (overlap(outs[x], outs[y])) return MHA_EINVAL;
    if (empty) {
        // Every gradient is a sum over no query rows.
        hipError_t e = hipSuccess;
        for (float* p : {dw_q, dw_k, dw_v, dw_o})
            if (e == hipSuccess) e = mha::launch_zero_f32(p, (long long)D * D, s);
        if (all_db)
            for (float* p : {db_q, db_k, db_v, db_o})
                if (e == hipSuccess) e = mha::launch_zero_f32(p, D, s);
        if (dx_kv && e == hipSuccess) e = mha::launch_zero_f32(dx_kv, (long long)B * Lk * D, s);
        return hip_status(e);
    }

    const void* ptrs[] = {x_q, x_kv, w_q, w_k, w_v, w_o, dout, workspace, b_q, b_k, b_v};
    for (int x = 0; x < 11; ++x) {
        if (!ptrs[x] && x < 8) return MHA_EINVAL;
        if (ptrs[x] && !aligned16(ptrs[x])) return MHA_EINVAL;
    }
    if (use_saved && (!saved || !aligned16(saved))) return MHA_EINVAL;
    const SavedLayout SL = saved_layout(B, Lq, Lk, D, h);
    if (use_saved && saved_bytes < SL.total) return MHA_EWORKSPACE;
    const BwdLayout L = bwd_layout(B, Lq, Lk, D, h, !use_saved);
    if (workspace_bytes < L.total) return MHA_EWORKSPACE;
    const size_t dw2 = (size_t)D * D * 2;
    const Range ins[] = {rng(x_q, (size_t)B * Lq * D * 2), rng(x_kv, (size_t)B * Lk * D * 2), rng(w_q, dw2),
                         rng(w_k, dw2), rng(w_v, dw2), rng(w_o, dw2), rng(dout, (size_t)B * Lq * D * 2),
                         rng(b_q, b_q ? (size_t)D * 2 : 0), rng(b_k, b_k ? (size_t)D * 2 : 0),
                         rng(b_v, b_v ? (size_t)D * 2 : 0)};
    const Range rws = rng(workspace, L.total);
    const Range rsv = rng(saved, use_saved ? SL.total : 0);
    for (int x = 0; x < n_out; ++x) {
        if (overlap(outs[x], rws) || overlap(outs[x], rsv)) return MHA_EINVAL;
        for (const Range& r : ins)
            if (overlap(outs[x], r)) return MHA_EINVAL;
    }
    for (const Range& r : ins)
        if (overlap(rws, r)) return MHA_EINVAL;
    if (overlap(rws, rsv)) return MHA_EINVAL;

    using mha::bf16_t;
    char* w = static_cast<char*>(workspace);
    // The forward's tensors: recomputed into the workspace, or the saved ones.
    char* fw = use_saved ? static_cast<char*>(const_cast<void*>(saved)) : w;
    const size_t oq = use_saved ? SL.q : L.q, ok = use_saved ? SL.k : L.k, ov = use_saved ? SL.v : L.v;
    const size_t oo = use_saved ? SL.ocat : L.ocat, ol = use_saved ? SL.lse : L.lse;
    bf16_t* Q = reinterpret_cast<bf16_t*>(fw + oq);
    bf16_t* K = reinterpret_cast<bf16_t*>(fw + ok);
    bf16_t* V = reinterpret_cast<bf16_t*>(fw + ov);
    bf16_t* Ocat = reinterpret_cast<bf16_t*>(fw + oo);
    bf16_t* dOcat = reinterpret_cast<bf16_t*>(w + L.docat);
    float* lse = reinterpret_cast<float*>(fw + ol);
    bf16_t* dQ = reinterpret_cast<bf16_t*>(w + L.dqkv);
    // [dK | dV]: right of dQ in the [M, 3D] block, or its own [Mk, 2D] block.
    bf16_t* dKV = fused_dx ? dQ + D : reinterpret_cast<bf16_t*>(w + L.dkv);
    const long long ld_q = fused_dx ? 3 * D : D, ld_kv = fused_dx ? 3 * D : 2 * D;
    bf16_t* WoT = reinterpret_cast<bf16_t*>(w + L.wt);
    bf16_t* WqT = WoT + (size_t)D * D;              // [D, 3D] (fused) or [D, D]
    bf16_t* WkvT = WoT + (size_t)2 * D * D;         // [D, 2D] (apart)
    const uint16_t* xq16 = static_cast<const uint16_t*>(x_q);
    const uint16_t* xkv16 = static_cast<const uint16_t*>(x_kv);
    hipError_t e;

    // 1. Transposed weights: dOcat = dout W_o and dx = dQ W_q + ... are
    // products with W (not W^T), which the GEMM takes as [N, K] = W^T.
    mha::TransposeArgs t;
    t.n = D;
    t.count = 4;
    t.w[0] = static_cast<const uint16_t*>(w_o); t.dst[0] = WoT; t.col0[0] = 0; t.ld[0] = D;
    t.w[1] = static_cast<const uint16_t*>(w_q);
    t.w[2] = static_cast<const uint16_t*>(w_k);
    t.w[3] = static_cast<const uint16_t*>(w_v);
    if (fused_dx) {
        for (int x = 1; x < 4; ++x) { t.dst[x] = WqT; t.col0[x] = (x - 1) * D; t.ld[x] = 3 * D; }
    } else {
        t.dst[1] = WqT; t.col0[1] = 0; t.ld[1] = D;
        t.dst[2] = WkvT; t.col0[2] = 0; t.ld[2] = 2 * D;
        t.dst[3] = WkvT; t.col0[3] = D; t.ld[3] = 2 * D;
    }
    e = timed("bwd_transpose_w", s, [&] { return mha::launch_transpose_bf16(t, s); });
    if (e != hipSuccess) return MHA_EHIP;

    if (!use_saved) {
    // 2. The forward's Q, K, V (bf16) in one launch.
    mha::GemmArgs g;
    g.nprob = 3;
    g.N = D;
    g.K = D;
    g.p[0] = {x_q, w_q, b_q, Q, B * Lq};
    g.p[1] = {x_kv, w_k, b_k, K, B * Lk};
    g.p[2] = {x_kv, w_v, b_v, V, B * Lk};
    e = timed("bwd_qkv_proj", s, [&] { return mha::launch_gemm_bf16(g, false, s); });
    if (e != hipSuccess) return MHA_EHIP;

    // 3. Attention forward on the head views: merged heads and log-sum-exp.
    mha::SdpaArgs a;
    a.q = Q; a.k = K; a.v = V; a.o = Ocat;
    a.sq[0] = (long long)Lq * D; a.sq[1] = kHeadDim; a.sq[2] = D;
    a.sk[0] = (long long)Lk * D; a.sk[1] = kHeadDim; a.sk[2] = D;
    a.sv[0] = (long long)Lk * D; a.sv[1] = kHeadDim; a.sv[2] = D;
    a.so[0] = (long long)Lq * D; a.so[1] = kHeadDim; a.so[2] = D;
    a.B = B; a.H = h; a.Lq = Lq; a.Lk = Lk;
    a.valid_lens = valid_lens;
    a.causal = causal ? 1 : 0;
    a.lse = lse;
    e = timed("bwd_attn_forward", s, [&] { return mha::launch_sdpa_bf16(a, false, s); });
    if (e != hipSuccess) return MHA_EHIP;
    }

    // 4. dOcat = dout W_o (bf16).
    mha::GemmArgs go;
    go.nprob = 1;
    go.N = D;
    go.K = D;
    go.p[0] = {dout, WoT, nullptr, dOcat, B * Lq};
    e = timed("bwd_out_proj", s, [&] { return mha::launch_gemm_bf16(go, false, s); });
    if (e != hipSuccess) return MHA_EHIP;

    // 5. Attention backward: dQ, dK, dV (bf16) beside each other.
    mha::BackwardArgs ba;
    ba.q = Q; ba.k = K; ba.v = V; ba.o = Ocat; ba.dout = dOcat;
    ba.dq = dQ; ba.dk = dKV; ba.dv = dKV + D;
    const long long lq_rows[3] = {(long long)Lq * D, kHeadDim, D}, lk_rows[3] = {(long long)Lk * D, kHeadDim, D};
    for (int x = 0; x < 3; ++x) {
        ba.sq[x] = lq_rows[x]; ba.so[x] = lq_rows[x]; ba.sdo[x] = lq_rows[x];
        ba.sk[x] = lk_rows[x]; ba.sv[x] = lk_rows[x];
    }
    ba.sdq[0] = (long long)Lq * ld_q; ba.sdq[1] = kHeadDim; ba.sdq[2] = ld_q;
    ba.sdk[0] = (long long)Lk * ld_kv; ba.sdk[1] = kHeadDim; ba.sdk[2] = ld_kv;
    for (int x = 0; x < 3; ++x) ba.sdv[x] = ba.sdk[x];
    ba.B = B; ba.H = h; ba.Lq = Lq; ba.Lk = Lk;
    ba.valid_lens = valid_lens;
    ba.vl_rank = valid_lens ? 1 : 0;
    ba.causal = causal ? 1 : 0;
    ba.in_f32 = false;
    ba.out_f32 = false;
    ba.rows = reinterpret_cast<float*>(w + L.rows);
    ba.lse_in = lse;
    e = timed("bwd_attn", s, [&] { return mha::launch_sdpa_backward(ba, s); });
    if (e != hipSuccess) return MHA_EHIP;

    // 6. Input gradients (fp32).
    mha::GemmArgs gx;
    gx.nprob = 1;
    gx.N = D;
    if (fused_dx) {
        gx.K = 3 * D;
        gx.p[0] = {dQ, WqT, nullptr, dx_q, B * Lq};
        e = timed("bwd_dx", s, [&] { return mha::launch_gemm_bf16(gx, true, s); });
    } else {
        gx.K = D;
        gx.p[0] = {dQ, WqT, nullptr, dx_q, B * Lq};
        e = timed("bwd_dx_q", s, [&] { return mha::launch_gemm_bf16(gx, true, s); });
        if (e != hipSuccess) return MHA_EHIP;
        gx.K = 2 * D;
        gx.p[0] = {dKV, WkvT, nullptr, dx_kv, B * Lk};
        e = timed("bwd_dx_kv", s, [&] { return mha::launch_gemm_bf16(gx, true, s); });
    }
    if (e != hipSuccess) return MHA_EHIP;

    // 7. Weight and bias gradients: dW_o = dout^T Ocat, dW_q = dQ^T x_q and
    // [dW_k; dW_v] = [dK | dV]^T x_kv, one launch pair.
    mha::TnArgs tn;
    tn.nprob = 3;
    tn.p[0].y = static_cast<const uint16_t*>(dout); tn.p[0].ldy = D;
    tn.p[0].x = Ocat; tn.p[0].ldx = D;
    tn.p[0].M = B * Lq; tn.p[0].N1 = D; tn.p[0].N2 = D;
    tn.p[0].dw = dw_o; tn.p[0].db = db_o;
    tn.p[1].y = dQ; tn.p[1].ldy = ld_q;
    tn.p[1].x = xq16; tn.p[1].ldx = D;
    tn.p[1].M = B * Lq; tn.p[1].N1 = D; tn.p[1].N2 = D;
    tn.p[1].dw = dw_q; tn.p[1].db = db_q;
    tn.p[2].y = dKV; tn.p[2].ldy = ld_kv;
    tn.p[2].x = xkv16; tn.p[2].ldx = D;
    tn.p[2].M = B * Lk; tn.p[2].N1 = 2 * D; tn.p[2].N2 = D;
    tn.p[2].dw = dw_k; tn.p[2].db = db_k;
    tn.p[2].dw2 = dw_v; tn.p[2].db2 = db_v;
    e = timed("bwd_dw", s, [&] { return mha::launch_gemm_tn(tn, w + L.tn, s); });
    return hip_status(e);
}

}  // namespace

extern "C" {

size_t mha_backward_workspace_bytes(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h) {
    if (in_dt != MHA_BF16 || !mha_train_sizes_ok(B, Lq, Lk, d_model, h)) return 0;
    return bwd_layout(B, Lq, Lk, d_model, h).total;
}

size_t mha_backward_saved_workspace_bytes(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h) {
    if (in_dt != MHA_BF16 || !mha_train_sizes_ok(B, Lq, Lk, d_model, h)) return 0;
    return bwd_layout(B, Lq, Lk, d_model, h, false).total;
}

size_t mha_saved_bytes(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h) {
    if (in_dt != MHA_BF16 || !mha_train_sizes_ok(B, Lq, Lk, d_model, h)) return 0;
    return saved_layout(B, Lq, Lk, d_model, h).total;
}

mha_status mha_backward(mha_dtype in_dt,
                        const void* x_q, const void* x_kv,
                        const void* w_q, const void* b_q,
                        const void* w_k, const void* b_k,
                        const void* w_v, const void* b_v,
                        const void* w_o,
                        const void* dout,
                        float* dx_q, float* dx_kv,
                        float* dw_q, float* db_q,
                        float* dw_k, float* db_k,
                        float* dw_v, float* db_v,
                        float* dw_o, float* db_o,
                        int B, int Lq, int Lk, int d_model, int h, int d_k,
                        const int* valid_lens, int causal,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return mha_backward_impl(in_dt, x_q, x_kv, w_q, b_q, w_k, b_k, w_v, b_v, w_o, nullptr, 0, dout, dx_q, dx_kv,
                             dw_q, db_q, dw_k, db_k, dw_v, db_v, dw_o, db_o, B, Lq, Lk, d_model, h, d_k, valid_lens,
                             causal, workspace, workspace_bytes, stream, false);
}

mha_status mha_backward_saved(mha_dtype in_dt,
                              const void* x_q, const void* x_kv,
                              const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                              const void* saved, size_t saved_bytes,
                              const void* dout,
                              float* dx_q, float* dx_kv,
                              float* dw_q, float* db_q,
                              float* dw_k, float* db_k,
                              float* dw_v, float* db_v,
                              float* dw_o, float* db_o,
                              int B, int Lq, int Lk, int d_model, int h, int d_k,
                              const int* valid_lens, int causal,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return mha_backward_impl(in_dt, x_q, x_kv, w_q, nullptr, w_k, nullptr, w_v, nullptr, w_o, saved, saved_bytes, dout,
                             dx_q, dx_kv, dw_q, db_q, dw_k, db_k, dw_v, db_v, dw_o, db_o, B, Lq, Lk, d_model, h, d_k,
                             valid_lens, causal, workspace, workspace_bytes, stream, true);
}

mha_status mha_forward_train(mha_dtype in_dt, mha_dtype out_dt,
                             const void* x_q, const void* x_kv,
                             const void* w_q, const void* b_q,
                             const void* w_k, const void* b_k,
                             const void* w_v, const void* b_v,
                             const void* w_o, const void* b_o,
                             void* out,
                             int B, int Lq, int Lk, int d_model, int h, int d_k,
                             const int* valid_lens, int causal,
                             void* saved, size_t saved_bytes, void* stream) {
    if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return MHA_EINVAL;
    if (B < 0 || Lq < 0 || Lk <= 0 || d_model <= 0 || h <= 0 || d_k <= 0) return MHA_EINVAL;
    if ((long long)h * d_k != d_model) return MHA_EINVAL;
    if (causal && Lq != Lk) return MHA_EINVAL;
    if (d_k != kHeadDim || in_dt != MHA_BF16) return MHA_ENOTSUP;
    if (!mha_train_sizes_ok(B, Lq, Lk, d_model, h)) return MHA_ENOTSUP;
    if (B == 0 || Lq == 0) return MHA_OK;
    const int D = d_model;
    const void* ptrs[] = {x_q, x_kv, w_q, w_k, w_v, w_o, out, saved, b_q, b_k, b_v, b_o};
    for (int x = 0; x < 12; ++x) {
        if (!ptrs[x] && x < 8) return MHA_EINVAL;
        if (ptrs[x] && !aligned16(ptrs[x])) return MHA_EINVAL;
    }
    const SavedLayout SL = saved_layout(B, Lq, Lk, D, h);
    if (saved_bytes < SL.total) return MHA_EWORKSPACE;
    auto rng = [](const void* p, size_t n) {
        const uintptr_t b = reinterpret_cast<uintptr_t>(p);
        return Range{b, b + n};
    };
    const size_t dw2 = (size_t)D * D * 2;
    const Range ins[] = {rng(x_q, (size_t)B * Lq * D * 2), rng(x_kv, (size_t)B * Lk * D * 2), rng(w_q, dw2),
                         rng(w_k, dw2), rng(w_v, dw2), rng(w_o, dw2), rng(b_q, b_q ? (size_t)D * 2 : 0),
                         rng(b_k, b_k ? (size_t)D * 2 : 0), rng(b_v, b_v ? (size_t)D * 2 : 0),
                         rng(b_o, b_o ? (size_t)D * 2 : 0)};
    const Range rout = rng(out, (size_t)B * Lq * D * elem_size(out_dt)), rsv = rng(saved, SL.total);
    if (overlap(rout, rsv)) return MHA_EINVAL;
    for (const Range& r : ins)
        if (overlap(rout, r) || overlap(rsv, r)) return MHA_EINVAL;

    using mha::bf16_t;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* sv = static_cast<char*>(saved);
    bf16_t* Q = reinterpret_cast<bf16_t*>(sv + SL.q);
    bf16_t* K = reinterpret_cast<bf16_t*>(sv + SL.k);
    bf16_t* V = reinterpret_cast<bf16_t*>(sv + SL.v);
    bf16_t* Ocat = reinterpret_cast<bf16_t*>(sv + SL.ocat);
    float* lse = reinterpret_cast<float*>(sv + SL.lse);
    hipError_t e;
    // 1. Q, K, V (bf16) in one launch.
    mha::GemmArgs g;
    g.nprob = 3;
    g.N = D;
    g.K = D;
    g.p[0] = {x_q, w_q, b_q, Q, B * Lq};
    g.p[1] = {x_kv, w_k, b_k, K, B * Lk};
    g.p[2] = {x_kv, w_v, b_v, V, B * Lk};
    e = timed("train_qkv_proj", s, [&] { return mha::launch_gemm_bf16(g, false, s); });
    if (e != hipSuccess) return MHA_EHIP;
    // 2. Attention on the head views: merged heads and log-sum-exp.
    mha::SdpaArgs a;
    a.q = Q; a.k = K; a.v = V; a.o = Ocat;
    a.sq[0] = (long long)Lq * D; a.sq[1] = kHeadDim; a.sq[2] = D;
    a.sk[0] = (long long)Lk * D; a.sk[1] = kHeadDim; a.sk[2] = D;
    a.sv[0] = (long long)Lk * D; a.sv[1] = kHeadDim; a.sv[2] = D;
    a.so[0] = (long long)Lq * D; a.so[1] = kHeadDim; a.so[2] = D;
    a.B = B; a.H = h; a.Lq = Lq; a.Lk = Lk;
    a.valid_lens = valid_lens;
    a.causal = causal ? 1 : 0;
    a.lse = lse;
    e = timed("train_attn", s, [&] { return mha::launch_sdpa_bf16(a, false, s); });
    if (e != hipSuccess) return MHA_EHIP;
    // 3. Output projection.
    mha::GemmArgs go;
    go.nprob = 1;
    go.N = D;
    go.K = D;
    go.p[0] = {Ocat, w_o, b_o, out, B * Lq};
    e = timed("train_out_proj", s, [&] { return mha::launch_gemm_bf16(go, out_dt == MHA_F32, s); });
    return hip_status(e);
}

size_t mha_sublayer_workspace_bytes(mha_dtype in_dt, int B, int L, int Lk, int d_model, int h) {
    const size_t inner = mha_workspace_bytes(in_dt, B, L, Lk, d_model, h);
    if (inner == 0 && !(B == 0 || L == 0)) return 0;
    if (!valid_dtype(in_dt) || B < 0 || L < 0 || d_model <= 0) return 0;
    return round_up((size_t)B * L * d_model * elem_size(in_dt), 256) + inner;
}

mha_status mha_sublayer_forward(mha_dtype in_dt, mha_dtype out_dt,
                                const void* x, const void* memory,
                                const void* ln_gain, const void* ln_bias, int ln_kind, float ln_eps,
                                const void* w_q, const void* b_q,
                                const void* w_k, const void* b_k,
                                const void* w_v, const void* b_v,
                                const void* w_o, const void* b_o,
                                void* out,
                                int B, int L, int Lk, int d_model, int h, int d_k,
                                const int* valid_lens, int causal,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return MHA_EINVAL;
    if (ln_kind != 0 && ln_kind != 1) return MHA_EINVAL;
    if (!(ln_eps >= 0.0f)) return MHA_EINVAL;
    if (!memory && Lk != L) return MHA_EINVAL;
    if (B < 0 || L < 0 || Lk <= 0 || d_model <= 1 || h <= 0 || d_k <= 0) return MHA_EINVAL;
    if ((long long)h * d_k != d_model) return MHA_EINVAL;
    if (d_k != kHeadDim) return MHA_ENOTSUP;
    if (in_dt == MHA_F32 && out_dt != MHA_F32) return MHA_ENOTSUP;
    if (B == 0 || L == 0) return MHA_OK;
    if (!mha_rows_fit(B, L, d_model) || !mha_rows_fit(B, Lk, d_model)) return MHA_ENOTSUP;
    if (!x || !out || !workspace) return MHA_EINVAL;
    const void* ptrs[] = {x, memory, ln_gain, ln_bias, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MHA_EINVAL;
    const size_t need = mha_sublayer_workspace_bytes(in_dt, B, L, Lk, d_model, h);
    if (need == 0) return MHA_EINVAL;
    if (workspace_bytes < need) return MHA_EWORKSPACE;
    const size_t ie = elem_size(in_dt);
    const size_t xbytes = round_up((size_t)B * L * d_model * ie, 256);
    const uintptr_t xb = reinterpret_cast<uintptr_t>(x), wb = reinterpret_cast<uintptr_t>(workspace);
    const Range rx{xb, xb + (size_t)B * L * d_model * ie}, rws{wb, wb + need};
    const uintptr_t ob = reinterpret_cast<uintptr_t>(out);
    const Range rout{ob, ob + (size_t)B * L * d_model * elem_size(out_dt)};
    if (overlap(rx, rws) || overlap(rx, rout)) return MHA_EINVAL;
    if (memory) {
        const uintptr_t mb = reinterpret_cast<uintptr_t>(memory);
        const Range rm{mb, mb + (size_t)B * Lk * d_model * ie};
        if (overlap(rm, rws) || overlap(rm, rout)) return MHA_EINVAL;
    }
    for (const void* p : {ln_gain, ln_bias}) {
        if (!p) continue;
        const Range r{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + (size_t)d_model * ie};
        if (overlap(r, rws) || overlap(r, rout)) return MHA_EINVAL;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    // norm(x) goes to the workspace (one row-wise pass), then the attention
    // layer runs on it with x as the residual of its output projection.
    void* xn = workspace;
    const hipError_t e = timed("layer_norm", s, [&] {
        return mha::launch_layer_norm(x, ln_gain, ln_bias, xn, B * L, d_model, ln_kind, ln_eps, in_dt == MHA_F32, s);
    });
    if (e != hipSuccess) return MHA_EHIP;
    return mha_impl(in_dt, out_dt, xn, memory ? memory : xn, w_q, b_q, w_k, b_k, w_v, b_v, w_o, b_o, out, B, L, Lk,
                    d_model, h, d_k, valid_lens, 1, causal, nullptr, mha_strides{0, 0, 0},
                    static_cast<char*>(workspace) + xbytes, need - xbytes, stream, x);
}

mha_status mha_timing_enable(int repeat) {
    if (repeat < 0 || repeat > 1000) return MHA_EINVAL;
    TimingState* t = t_timing;
    if (repeat == 0) {
        if (t) t->on = false;
        return MHA_OK;
    }
    if (!t) {
        t = new (std::nothrow) TimingState();
        if (!t) return MHA_EHIP;
        for (int n = 0; n < 2 * kPool; ++n) {
            if (hipEventCreate(&t->ev[n]) != hipSuccess) {
                for (int x = 0; x < n; ++x) (void)hipEventDestroy(t->ev[x]);
                delete t;
                return MHA_EHIP;
            }
        }
        t_timing = t;
    }
    t->on = true;
    t->repeat = repeat;
    return MHA_OK;
}

int mha_timing_read(const char** names, double* total_ms, int* count, int max) {
    TimingState* t = t_timing;
    if (!t) return 0;
    int n_out = 0;
    for (int k = 0; k < t->used; ++k) {
        if (hipEventSynchronize(t->ev[2 * k + 1]) != hipSuccess) return -1;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, t->ev[2 * k], t->ev[2 * k + 1]) != hipSuccess) return -1;
        int slot = -1;
        for (int x = 0; x < n_out; ++x)
            if (strcmp(names[x], t->name[k]) == 0) slot = x;
        if (slot < 0) {
            if (n_out >= max) continue;
            slot = n_out++;
            names[slot] = t->name[k];
            total_ms[slot] = 0.0;
            count[slot] = 0;
        }
        total_ms[slot] += ms;
        count[slot] += t->repeat;
    }
    t->used = 0;
    return n_out;
}

}  // extern "C"
