// C ABI of libattn.so: argument validation, workspace sizing and dispatch.
// Every check runs before the first HIP call; nothing here allocates, frees or
// synchronises.
#include <math.h>

#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/attn.h"
#include "attn_internal.h"

using namespace attn;

namespace {

thread_local std::string g_last_error;
thread_local TimingHook g_timing;

// Takes (and clears) this thread's timing hook.
TimingHook take_timing() {
  TimingHook t = g_timing;
  g_timing = TimingHook();
  return t;
}

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return ATTN_OK;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool supported_hd(int hd) { return hd == 8 || hd == 16 || hd == 32 || hd == 64 || hd == 128; }

size_t elem_bytes(int dtype) { return dtype == ATTN_DTYPE_BF16 ? 2 : 4; }

// 4 theta_i / (2 pi) = base^(-2i/hd) * 2 / pi in fp64: quarter turns per position.
RopeFreqs make_freqs(int hd, double base) {
  RopeFreqs f;
  memset(&f, 0, sizeof(f));
  if (base != 0.0) {
    for (int i = 0; i < hd / 2; ++i) f.rev[i] = pow(base, -2.0 * i / hd) * (2.0 / M_PI);
  }
  return f;
}

int check_common(int dtype, int out_dtype, int alibi, double rope_base, int hd) {
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (out_dtype != ATTN_DTYPE_F32 && out_dtype != ATTN_DTYPE_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if (alibi < ATTN_ALIBI_NONE || alibi > ATTN_ALIBI_PAGE1) return fail(ATTN_ERR_UNSUPPORTED, "alibi %d", alibi);
  if (!(rope_base >= 0.0) || !isfinite(rope_base) || (rope_base > 0.0 && rope_base <= 1.0))
    return fail(ATTN_ERR_UNSUPPORTED, "rope_base %g (0 disables, otherwise > 1)", rope_base);
  if (hd <= 0 || hd % 2) return fail(ATTN_ERR_SHAPE, "head dim %d must be positive and even", hd);
  if (!supported_hd(hd)) return fail(ATTN_ERR_UNSUPPORTED, "head dim %d not in {8,16,32,64,128}", hd);
  return ATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr long long kMaxElems = 1LL << 40;

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_set_timing_events(void* start, void* stop) {
  g_timing.start = reinterpret_cast<hipEvent_t>(start);
  g_timing.stop = reinterpret_cast<hipEvent_t>(stop);
  return ATTN_OK;
}

size_t attn_prefill_workspace_bytes(int B, int T, int KV, int hd, int dtype, double rope_base) {
  if (B <= 0 || T <= 0 || KV <= 0 || hd <= 0 || rope_base == 0.0) return 0;
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return 0;
  const long long n = (long long)B * KV * T * hd;
  if (n > kMaxElems) return 0;
  return (size_t)n * elem_bytes(dtype);
}

}  // extern "C"

namespace {

// Shared body of both prefill entry points: Tq query rows that are key tokens
// q_off .. q_off+Tq-1 of a Tk-token sequence, optional sliding window.
int prefill_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Tq, int Tk, int H,
                 int KV, int hd, int pos0, int q_off, int window, double rope_base, int causal, int alibi,
                 int dtype, int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !out) return fail(ATTN_ERR_NULL, "q, k, v and out must be non-NULL");
  if (B <= 0 || Tq <= 0 || Tk <= 0 || H <= 0 || KV <= 0)
    return fail(ATTN_ERR_SHAPE, "sizes must be positive (B=%d Tq=%d Tk=%d H=%d KV=%d)", B, Tq, Tk, H, KV);
  if (H % KV) return fail(ATTN_ERR_SHAPE, "H=%d is not a multiple of KV=%d", H, KV);
  if (q_off < 0 || (long long)q_off + Tq > Tk)
    return fail(ATTN_ERR_SHAPE, "query chunk [%d, %d) must lie inside the %d keys", q_off, q_off + Tq, Tk);
  if (pos0 < 0 || (long long)pos0 + Tk > 0x7fffffffLL) return fail(ATTN_ERR_SHAPE, "pos0=%d out of range", pos0);
  if (H > 65535 || B > 65535 || (long long)B * KV > 65535 * 8LL)
    return fail(ATTN_ERR_SHAPE, "H, B and B*KV/8 must be <= 65535");
  if (int c = check_common(dtype, out_dtype, alibi, rope_base, hd)) return c;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_UNSUPPORTED, "causal %d", causal);
  if (window < 0) return fail(ATTN_ERR_SHAPE, "window %d must be >= 0", window);
  if (window > 0 && !causal) return fail(ATTN_ERR_UNSUPPORTED, "a sliding window needs causal attention");
  if ((long long)B * H * Tq * hd > kMaxElems || (long long)B * KV * Tk * hd > kMaxElems)
    return fail(ATTN_ERR_SHAPE, "tensor too large");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(ATTN_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(ATTN_ERR_ALIGN, "lse must be 4-byte aligned");
  const size_t need = attn_prefill_workspace_bytes(B, Tk, KV, hd, dtype, rope_base);
  if (need) {
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (workspace_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
  }

  const int bf16 = dtype == ATTN_DTYPE_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.Tq = Tq;
  a.Tk = Tk;
  a.H = H;
  a.KV = KV;
  a.hd = hd;
  a.group = H / KV;
  a.pos0 = pos0;
  a.q_off = q_off;
  // a window covering every key a query can see changes nothing
  a.window = (window > 0 && window < q_off + Tq) ? window : 0;
  a.causal = causal;
  a.rope = rope_base != 0.0;
  a.alibi = alibi;
  a.out_bf16 = out_dtype == ATTN_DTYPE_BF16;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
  a.freqs = make_freqs(hd, rope_base);

  if (a.rope) {
    RopeKArgs r;
    r.k = k;
    r.kr = workspace;
    r.heads = B * KV;
    r.T = Tk;
    r.hd = hd;
    r.pos0 = pos0;
    r.freqs = a.freqs;
    if (int c = hip_status(launch_rope_k(r, bf16, s), "rope_k launch")) return c;
    a.k = workspace;
  }
  const TimingHook tm = take_timing();
  if (int c = hip_status(tm.before(s), "timing event")) return c;
  if (prefill_mfma_supported(a, bf16)) {
    if (int c = hip_status(launch_prefill_mfma(a, s), "prefill_mfma launch")) return c;
  } else {
    if (int c = hip_status(launch_prefill_valu(a, bf16, s), "prefill_valu launch")) return c;
  }
  return hip_status(tm.after(s), "timing event");
}

}  // namespace

extern "C" {

int attn_prefill_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int T, int H,
                     int KV, int hd, int pos0, double rope_base, int causal, int alibi, int dtype, int out_dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k, v, out, lse, B, T, T, H, KV, hd, pos0, 0, 0, rope_base, causal, alibi, dtype, out_dtype,
                      workspace, workspace_bytes, stream);
}

int attn_prefill_ex_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Tq, int Tk,
                        int H, int KV, int hd, int pos0, int q_offset, int window, double rope_base, int causal,
                        int alibi, int dtype, int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k, v, out, lse, B, Tq, Tk, H, KV, hd, pos0, q_offset, window, rope_base, causal, alibi,
                      dtype, out_dtype, workspace, workspace_bytes, stream);
}

namespace {
// Backward workspace: [rotated K][rotated Q][D fp32], each region 256-byte
// aligned; the rotated copies exist only when RoPE is on.
struct BwdWs {
  long long kr, qr, d, total;
};
BwdWs bwd_ws_layout(int B, int T, int H, int KV, int hd, int dtype, double rope_base) {
  const auto up = [](long long n) { return (n + 255) / 256 * 256; };
  const long long eb = elem_bytes(dtype);
  const long long nk = rope_base != 0.0 ? (long long)B * KV * T * hd * eb : 0;
  const long long nq = rope_base != 0.0 ? (long long)B * H * T * hd * eb : 0;
  BwdWs w;
  w.kr = 0;
  w.qr = up(nk);
  w.d = w.qr + up(nq);
  w.total = w.d + up((long long)B * H * T * 4);
  return w;
}
}  // namespace

size_t attn_prefill_bwd_workspace_bytes(int B, int T, int H, int KV, int hd, int dtype, double rope_base) {
  if (B <= 0 || T <= 0 || H <= 0 || KV <= 0 || hd <= 0) return 0;
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return 0;
  if ((long long)B * H * T * hd > kMaxElems) return 0;
  return (size_t)bwd_ws_layout(B, T, H, KV, hd, dtype, rope_base).total;
}

int attn_prefill_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int T, int H, int KV, int hd, int pos0,
                     double rope_base, int causal, int alibi, int dtype, int out_dtype, int grad_dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv)
    return fail(ATTN_ERR_NULL, "q, k, v, out, lse, dout, dq, dk and dv must be non-NULL");
  if (B <= 0 || T <= 0 || H <= 0 || KV <= 0)
    return fail(ATTN_ERR_SHAPE, "sizes must be positive (B=%d T=%d H=%d KV=%d)", B, T, H, KV);
  if (H % KV) return fail(ATTN_ERR_SHAPE, "H=%d is not a multiple of KV=%d", H, KV);
  if (pos0 < 0 || (long long)pos0 + T > 0x7fffffffLL) return fail(ATTN_ERR_SHAPE, "pos0=%d out of range", pos0);
  if (H > 65535 || B > 65535 || KV > 65535) return fail(ATTN_ERR_SHAPE, "H, KV and B must be <= 65535");
  if (int c = check_common(dtype, out_dtype, alibi, rope_base, hd)) return c;
  if (grad_dtype != ATTN_DTYPE_F32 && grad_dtype != ATTN_DTYPE_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "grad_dtype %d", grad_dtype);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_UNSUPPORTED, "causal %d", causal);
  if ((long long)B * H * T * hd > kMaxElems) return fail(ATTN_ERR_SHAPE, "tensor too large");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(ATTN_ERR_ALIGN, "tensors must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(ATTN_ERR_ALIGN, "lse must be 4-byte aligned");
  const BwdWs lay = bwd_ws_layout(B, T, H, KV, hd, dtype, rope_base);
  if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace of %lld bytes required", lay.total);
  if (workspace_bytes < (size_t)lay.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes < required %lld", workspace_bytes, lay.total);
  if (!aligned(workspace, 256)) return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  const int bf16 = dtype == ATTN_DTYPE_BF16;
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.out = out;
  a.lse = lse;
  a.D = reinterpret_cast<float*>(ws + lay.d);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.T = T;
  a.H = H;
  a.KV = KV;
  a.hd = hd;
  a.group = H / KV;
  a.pos0 = pos0;
  a.causal = causal;
  a.rope = rope_base != 0.0;
  a.alibi = alibi;
  a.in_bf16 = bf16;
  a.out_bf16 = out_dtype == ATTN_DTYPE_BF16;
  a.grad_bf16 = grad_dtype == ATTN_DTYPE_BF16;
  a.scale = (float)(1.0 / sqrt((double)hd));
  a.freqs = make_freqs(hd, rope_base);

  if (a.rope) {  // rotated copies of K and Q, written once
    RopeKArgs r;
    memset(&r, 0, sizeof(r));
    r.hd = hd;
    r.T = T;
    r.pos0 = pos0;
    r.freqs = a.freqs;
    r.k = k;
    r.kr = ws + lay.kr;
    r.heads = B * KV;
    if (int c = hip_status(launch_rope_k(r, bf16, s), "rope_k launch")) return c;
    r.k = q;
    r.kr = ws + lay.qr;
    r.heads = B * H;
    if (int c = hip_status(launch_rope_k(r, bf16, s), "rope_q launch")) return c;
    a.k = ws + lay.kr;
    a.q = ws + lay.qr;
  }
  const TimingHook tm = take_timing();
  // the matrix-core dq kernel computes D itself (its rows' dout are already in
  // registers); the vector-ALU kernels take it from a pre-pass
  if (bwd_mfma_supported(a)) return hip_status(launch_bwd_mfma(a, s, tm), "backward launch");
  BwdPrepArgs pa;
  pa.out = out;
  pa.dout = dout;
  pa.D = reinterpret_cast<float*>(ws + lay.d);
  pa.rows = (long)B * H * T;
  pa.hd = hd;
  pa.out_bf16 = a.out_bf16;
  if (int c = hip_status(launch_bwd_prep(pa, s), "backward prep launch")) return c;
  if (int c = hip_status(tm.before(s), "timing event")) return c;
  if (int c = hip_status(launch_bwd_valu(a, s), "backward launch")) return c;
  return hip_status(tm.after(s), "timing event");
}

namespace {
// Workspace layout: [part_o: rows*hd fp32][part_ml: rows float2], rows =
// B*H*ceil(Lmax/split). The caller-owned workspace is sized for the smallest
// split (256 slots), so it fits whichever kernel runs.
struct DecodeWs {
  long long part_o, part_ml, total;
};
DecodeWs decode_ws_layout(int B, int H, int hd, int Lmax, int split = kDecodeSplit) {
  const long long rows = (long long)B * H * ((Lmax + split - 1) / split);
  DecodeWs w;
  w.part_o = 0;
  w.part_ml = rows * hd * 4;
  w.total = (w.part_ml + rows * 8 + 255) / 256 * 256;
  return w;
}
}  // namespace

size_t attn_decode_workspace_bytes(int B, int H, int KV, int hd, int Lmax) {
  if (B <= 0 || H <= 0 || KV <= 0 || hd <= 0 || Lmax <= 0) return 0;
  return (size_t)decode_ws_layout(B, H, hd, Lmax).total;
}

namespace {
// ---- scratch of the allocation-free decode entry point
// The split partials of attn_decode_fwd_noalloc live in this file-scope device
// array: one copy per GPU, created when the library's code object is loaded
// on that GPU and held until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: its device address on the current
// GPU comes from hipGetSymbolAddress, looked up once per device and kept.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
int scratch_ptr(void** out) {
  int dev = -1;
  if (int c = hip_status(hipGetDevice(&dev), "hipGetDevice")) return c;
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_ERR_HIP, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (int c = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) return c;
    if (!p) return fail(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

// Shared body of the decode entry points. noalloc: the partials go to the
// per-device scratch array instead of the caller's workspace.
int decode_impl(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                const int32_t* cache_lens, void* out, float* lse, int B, int H, int KV, int hd, int Lmax,
                double rope_base, int alibi, int dtype, int out_dtype, void* workspace, size_t workspace_bytes,
                void* stream, int fp8, float k_scale, float v_scale, bool noalloc = false) {
  if (!q || !k_cache || !v_cache || !cache_lens || !out)
    return fail(ATTN_ERR_NULL, "q, k_cache, v_cache, cache_lens and out must be non-NULL");
  // k_new and v_new both NULL: slot L already holds the new token (bf16/fp32 caches only)
  const bool append = k_new || v_new;
  if (append && (!k_new || !v_new)) return fail(ATTN_ERR_NULL, "k_new and v_new must both be given or both be NULL");
  if (!append && fp8) return fail(ATTN_ERR_NULL, "the fp8 cache needs k_new and v_new");
  if (B <= 0 || H <= 0 || KV <= 0 || Lmax <= 0)
    return fail(ATTN_ERR_SHAPE, "sizes must be positive (B=%d H=%d KV=%d Lmax=%d)", B, H, KV, Lmax);
  if (H % KV) return fail(ATTN_ERR_SHAPE, "H=%d is not a multiple of KV=%d", H, KV);
  if (H > 65535 || B > 65535 || KV > 65535) return fail(ATTN_ERR_SHAPE, "H, KV and B must be <= 65535");
  if (int c = check_common(dtype, out_dtype, alibi, rope_base, hd)) return c;
  if ((long long)B * KV * Lmax * hd > kMaxElems) return fail(ATTN_ERR_SHAPE, "cache too large");
  // (the split grid holds at most 65535 splits per sequence)
  if (Lmax > kMaxDecodeLmax) return fail(ATTN_ERR_SHAPE, "Lmax=%d exceeds %d cache slots", Lmax, kMaxDecodeLmax);
  if (!aligned(q, 16) || (append && (!aligned(k_new, 16) || !aligned(v_new, 16))) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(ATTN_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(cache_lens, 4) || (lse && !aligned(lse, 4)))
    return fail(ATTN_ERR_ALIGN, "cache_lens and lse must be 4-byte aligned");
  if (!noalloc) {
    const size_t need = attn_decode_workspace_bytes(B, H, KV, hd, Lmax);
    if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (workspace_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
  }

  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.lens = cache_lens;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.KV = KV;
  a.hd = hd;
  a.group = H / KV;
  a.Lmax = Lmax;
  a.fp8 = fp8;
  DecodeWs lay = decode_ws_layout(B, H, hd, Lmax);
  if (noalloc) {
    // sized for the split the launcher picks (checked before any HIP call)
    lay = decode_ws_layout(B, H, hd, Lmax, decode_split_for(a, dtype == ATTN_DTYPE_BF16));
    if ((unsigned long long)lay.total > kNoAllocScratchBytes)
      return fail(ATTN_ERR_WORKSPACE, "the step needs %lld bytes of partials; the allocation-free entry point holds %zu",
                  lay.total, kNoAllocScratchBytes);
  }
  if (!noalloc) {
    char* ws = reinterpret_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws + lay.part_o);
    a.part_ml = reinterpret_cast<float2*>(ws + lay.part_ml);
  }
  a.split = kDecodeSplit;  // the launcher sets the split of the kernel it picks
  a.nsplit = (Lmax + kDecodeSplit - 1) / kDecodeSplit;
  a.rope = rope_base != 0.0;
  a.alibi = alibi;
  a.out_bf16 = out_dtype == ATTN_DTYPE_BF16;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
  a.freqs = make_freqs(hd, rope_base);
  a.fp8 = fp8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.append = append;
  if (fp8) {
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
      return fail(ATTN_ERR_SHAPE, "k_scale and v_scale must be positive and finite (%g, %g)", (double)k_scale,
                  (double)v_scale);
    if (dtype != ATTN_DTYPE_BF16 || !decode_mfma_supported(a, 1))
      return fail(ATTN_ERR_UNSUPPORTED, "fp8 cache: bf16 q/k_new/v_new, hd 64 or 128 and H/KV <= 16 (got dtype %d, "
                                        "hd %d, H/KV %d)", dtype, hd, H / KV);
  }
  if (noalloc) {  // every argument is valid: now the one HIP call of the set-up
    void* p = nullptr;
    if (int c = scratch_ptr(&p)) return c;
    char* ws = reinterpret_cast<char*>(p);
    a.part_o = reinterpret_cast<float*>(ws + lay.part_o);
    a.part_ml = reinterpret_cast<float2*>(ws + lay.part_ml);
  }
  const TimingHook tm = take_timing();
  return hip_status(launch_decode(a, dtype == ATTN_DTYPE_BF16, reinterpret_cast<hipStream_t>(stream), tm),
                    "decode launch");
}
}  // namespace

namespace {
// Workspace of the latent decode: [folded queries bf16][partials fp32][(m, l)][merged latent outputs fp32]
// [work list of the split kernel].
struct LatentWs {
  long long qt, part_o, part_ml, ot, items, total;
};
LatentWs latent_ws_layout(int B, int H, int dc, int Lmax) {
  auto up = [](long long x) { return (x + 255) / 256 * 256; };
  const long long nsplit = (Lmax + kLatentSplit - 1) / kLatentSplit;
  const long long rows = (long long)B * H;
  LatentWs w;
  w.qt = 0;
  w.part_o = up(rows * dc * 2);
  w.part_ml = w.part_o + up(rows * nsplit * dc * 4);
  w.ot = w.part_ml + up(rows * nsplit * 8);
  w.items = w.ot + up(rows * dc * 4);
  w.total = w.items + up(((long long)B * nsplit + 1) * 4);
  return w;
}
}  // namespace

size_t attn_decode_latent_workspace_bytes(int B, int H, int dc, int Lmax) {
  if (B <= 0 || H <= 0 || dc <= 0 || Lmax <= 0) return 0;
  return (size_t)latent_ws_layout(B, H, dc, Lmax).total;
}

int attn_decode_latent_fwd(const void* q, const void* c_new, void* c_cache, const int32_t* cache_lens,
                           const void* w_uk, const void* w_uv, void* out, float* lse, int B, int H, int hd, int dc,
                           int Lmax, int alibi, int dtype, int out_dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!q || !c_new || !c_cache || !cache_lens || !w_uk || !w_uv || !out)
    return fail(ATTN_ERR_NULL, "q, c_new, c_cache, cache_lens, w_uk, w_uv and out must be non-NULL");
  if (B <= 0 || H <= 0 || Lmax <= 0 || hd <= 0 || dc <= 0)
    return fail(ATTN_ERR_SHAPE, "sizes must be positive (B=%d H=%d hd=%d dc=%d Lmax=%d)", B, H, hd, dc, Lmax);
  if (B > 65535 || H > 65535) return fail(ATTN_ERR_SHAPE, "B and H must be <= 65535");
  if (dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED, "latent decode takes bf16 inputs (dtype %d)", dtype);
  if (out_dtype != ATTN_DTYPE_F32 && out_dtype != ATTN_DTYPE_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if (hd != 64 && hd != 128) return fail(ATTN_ERR_UNSUPPORTED, "hd %d (supported: 64, 128)", hd);
  if (dc != 256 && dc != 512) return fail(ATTN_ERR_UNSUPPORTED, "latent width %d (supported: 256, 512)", dc);
  if (alibi < ATTN_ALIBI_NONE || alibi > ATTN_ALIBI_PAGE1) return fail(ATTN_ERR_UNSUPPORTED, "alibi %d", alibi);
  if ((Lmax + kLatentSplit - 1) / kLatentSplit > kLatentMaxSplits || (long long)Lmax * dc * 2 >= (1LL << 31))
    return fail(ATTN_ERR_SHAPE, "Lmax=%d too large for the latent cache", Lmax);
  if ((long long)B * Lmax * dc > kMaxElems) return fail(ATTN_ERR_SHAPE, "cache too large");
  if (!aligned(q, 16) || !aligned(c_new, 16) || !aligned(c_cache, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16) ||
      !aligned(out, 16))
    return fail(ATTN_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(cache_lens, 4) || (lse && !aligned(lse, 4)))
    return fail(ATTN_ERR_ALIGN, "cache_lens and lse must be 4-byte aligned");
  const LatentWs lay = latent_ws_layout(B, H, dc, Lmax);
  if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace of %lld bytes required", lay.total);
  if (workspace_bytes < (size_t)lay.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes < required %lld", workspace_bytes, lay.total);
  if (!aligned(workspace, 256)) return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");

  LatentArgs a;
  memset(&a, 0, sizeof(a));
  char* ws = reinterpret_cast<char*>(workspace);
  a.q = q;
  a.c_new = c_new;
  a.c_cache = c_cache;
  a.lens = cache_lens;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.out = out;
  a.lse = lse;
  a.qt = reinterpret_cast<uint16_t*>(ws + lay.qt);
  a.part_o = reinterpret_cast<float*>(ws + lay.part_o);
  a.part_ml = reinterpret_cast<float2*>(ws + lay.part_ml);
  a.ot = reinterpret_cast<float*>(ws + lay.ot);
  a.items = reinterpret_cast<int*>(ws + lay.items);
  a.B = B;
  a.H = H;
  a.hd = hd;
  a.dc = dc;
  a.Lmax = Lmax;
  a.hblocks = (H + 15) / 16;
  a.split = kLatentSplit;
  a.nsplit = (Lmax + kLatentSplit - 1) / kLatentSplit;
  a.alibi = alibi;
  a.out_bf16 = out_dtype == ATTN_DTYPE_BF16;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
  const TimingHook tm = take_timing();
  return hip_status(launch_decode_latent(a, reinterpret_cast<hipStream_t>(stream), tm), "latent decode launch");
}

int attn_decode_fwd(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* cache_lens, void* out, float* lse, int B, int H, int KV, int hd, int Lmax,
                    double rope_base, int alibi, int dtype, int out_dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_impl(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, B, H, KV, hd, Lmax, rope_base, alibi,
                     dtype, out_dtype, workspace, workspace_bytes, stream, 0, 1.f, 1.f);
}

int attn_decode_fwd_noalloc(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* cache_lens, void* out, float* lse, int B, int H, int KV, int hd, int Lmax,
                            double rope_base, int alibi, int dtype, int out_dtype, void* stream) {
  return decode_impl(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, B, H, KV, hd, Lmax, rope_base, alibi,
                     dtype, out_dtype, nullptr, 0, stream, 0, 1.f, 1.f, true);
}

int attn_decode_fp8_fwd(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* cache_lens, void* out, float* lse, int B, int H, int KV, int hd, int Lmax,
                        double rope_base, int alibi, float k_scale, float v_scale, int dtype, int out_dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, B, H, KV, hd, Lmax, rope_base, alibi,
                     dtype, out_dtype, workspace, workspace_bytes, stream, 1, k_scale, v_scale);
}

}  // extern "C"

// ------------------------------------------------------------------ projections
#include "proj_internal.h"

namespace {
// Checks shared by the projections; M = B*T rows of K inputs, N outputs.
int proj_checks(int B, int T, int H, int KV, int hd, int D, int dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || KV <= 0 || hd <= 0 || D <= 0)
    return fail(ATTN_ERR_SHAPE, "sizes must be positive (B=%d T=%d D=%d H=%d KV=%d hd=%d)", B, T, D, H, KV, hd);
  if (H % KV) return fail(ATTN_ERR_SHAPE, "H=%d is not a multiple of KV=%d", H, KV);
  if (hd % 2) return fail(ATTN_ERR_SHAPE, "head dim %d must be even", hd);
  if (dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED, "projections take bf16 (dtype %d)", dtype);
  if (hd != 64 && hd != 128) return fail(ATTN_ERR_UNSUPPORTED, "projections support head dim 64 or 128 (got %d)", hd);
  if (D % 64) return fail(ATTN_ERR_UNSUPPORTED, "model dim %d must be a multiple of 64", D);
  const long long M = (long long)B * T, N = (long long)(H + 2 * KV) * hd;
  if (M * D * 2 >= (1LL << 31) || N * D * 2 >= (1LL << 31) || M * H * hd * 2 >= (1LL << 31) ||
      (long long)D * H * hd * 2 >= (1LL << 31))
    return fail(ATTN_ERR_SHAPE, "every operand must be under 2 GiB");
  return ATTN_OK;
}

int qkv_impl(const void* x, const void* w, void* q, void* k, void* v, void* k_cache, void* v_cache,
             const int32_t* lens, int B, int T, int D, int H, int KV, int hd, int Lmax, int pos0, double rope_base,
             int dtype, void* stream, int mode) {
  if (int c = proj_checks(B, T, H, KV, hd, D, dtype)) return c;
  if (!(rope_base == 0.0 || rope_base > 1.0) || !std::isfinite(rope_base))
    return fail(ATTN_ERR_UNSUPPORTED, "rope_base %g (0 disables, otherwise > 1)", rope_base);
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 16)) return fail(ATTN_ERR_ALIGN, "tensors must be 16-byte aligned");
  ProjArgs a;
  memset(&a, 0, sizeof(a));
  if (mode == PROJ_QKV_CACHE) {
    if (Lmax <= 0 || T > Lmax) return fail(ATTN_ERR_SHAPE, "Lmax=%d must be positive and >= T=%d", Lmax, T);
    if ((long long)B * KV * Lmax * hd > kMaxElems) return fail(ATTN_ERR_SHAPE, "cache too large");
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(lens, 4))
      return fail(ATTN_ERR_ALIGN, "caches must be 16-byte aligned and cache_lens 4-byte aligned");
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.lens = lens;
    a.Lmax = Lmax;
  } else {
    if (pos0 < 0 || (long long)pos0 + T > 0x7fffffffLL) return fail(ATTN_ERR_SHAPE, "pos0=%d out of range", pos0);
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(ATTN_ERR_ALIGN, "tensors must be 16-byte aligned");
    a.k = k;
    a.v = v;
    a.pos0 = pos0;
  }
  a.a = x;
  a.w = w;
  a.M = B * T;
  a.N = (H + 2 * KV) * hd;
  a.K = D;
  a.T = T;
  a.H = H;
  a.KV = KV;
  a.hd = hd;
  a.a_bytes = (unsigned)((long long)a.M * D * 2);
  a.w_bytes = (unsigned)((long long)a.N * D * 2);
  a.q = q;
  a.rope = rope_base != 0.0;
  a.freqs = make_freqs(hd, rope_base);
  const TimingHook tm = take_timing();
  return hip_status(launch_proj(a, mode, reinterpret_cast<hipStream_t>(stream), tm), "projection launch");
}
}  // namespace

int attn_qkv_proj_fwd(const void* x, const void* w_qkv, void* q, void* k, void* v, int B, int T, int D, int H,
                      int KV, int hd, int pos0, double rope_base, int dtype, void* stream) {
  if (!x || !w_qkv || !q || !k || !v) return fail(ATTN_ERR_NULL, "x, w_qkv, q, k and v must be non-NULL");
  if (int c = qkv_impl(x, w_qkv, q, k, v, nullptr, nullptr, nullptr, B, T, D, H, KV, hd, 0, pos0, rope_base, dtype,
                       stream, PROJ_QKV))
    return c;
  return ok();
}

int attn_qkv_proj_cache_fwd(const void* x, const void* w_qkv, void* q, void* k_cache, void* v_cache,
                            const int32_t* cache_lens, int B, int T, int D, int H, int KV, int hd, int Lmax,
                            double rope_base, int dtype, void* stream) {
  if (!x || !w_qkv || !q || !k_cache || !v_cache || !cache_lens)
    return fail(ATTN_ERR_NULL, "x, w_qkv, q, k_cache, v_cache and cache_lens must be non-NULL");
  if (int c = qkv_impl(x, w_qkv, q, nullptr, nullptr, k_cache, v_cache, cache_lens, B, T, D, H, KV, hd, Lmax, 0,
                       rope_base, dtype, stream, PROJ_QKV_CACHE))
    return c;
  return ok();
}

int attn_out_proj_fwd(const void* o, const void* w_o, void* y, int B, int T, int H, int hd, int D, int dtype,
                      int out_dtype, void* stream) {
  if (!o || !w_o || !y) return fail(ATTN_ERR_NULL, "o, w_o and y must be non-NULL");
  if (int c = proj_checks(B, T, H, H, hd, D, dtype)) return c;
  if (out_dtype != ATTN_DTYPE_F32 && out_dtype != ATTN_DTYPE_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if ((long long)B * T * D * 4 >= (1LL << 31)) return fail(ATTN_ERR_SHAPE, "every operand must be under 2 GiB");
  if (!aligned(o, 16) || !aligned(w_o, 16) || !aligned(y, 16)) return fail(ATTN_ERR_ALIGN, "tensors must be 16-byte aligned");
  ProjArgs a;
  memset(&a, 0, sizeof(a));
  a.a = o;
  a.w = w_o;
  a.M = B * T;
  a.N = D;
  a.K = H * hd;
  a.T = T;
  a.H = H;
  a.KV = H;
  a.hd = hd;
  a.a_bytes = (unsigned)((long long)B * H * T * hd * 2);
  a.w_bytes = (unsigned)((long long)D * H * hd * 2);
  a.y = y;
  a.out_bf16 = out_dtype == ATTN_DTYPE_BF16;
  const TimingHook tm = take_timing();
  if (int c = hip_status(launch_proj(a, PROJ_OUT, reinterpret_cast<hipStream_t>(stream), tm), "projection launch"))
    return c;
  return ok();
}
