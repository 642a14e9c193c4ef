// C entry points: argument validation, then the launches on the caller's stream.
//
// Checks follow the op's rules as the pages state them: docs.rs page
// "onnx-runtime-ep-cuda src/kernels/paged_attention.rs", PagedAttentionFactory
// (attribute defaults), unsupported_reason and execute (block size a power of
// two >= 16, v_head_size in 1..=head_size, rotary_offset + rotary_dim <=
// head_size, explicit scale required when v_head_size != head_size, float16 /
// bfloat16 only, token_count * num_heads within grid limits); PR #1940
// "PagedAttention v1 audit and MLA oracle", third commit (rotary caches:
// head_size % 16 == 0, rotary_dim = 2 * cos_cache.shape[1] with
// cos_cache.shape[1] <= head_size / 2 and a multiple of 8); PR #1955 review
// (rotary_offset % 8 == 0, head_size % 8 == 0). The separate (grouped-query)
// layout adds the head-ratio rule of PR #1940's third commit (num_heads a
// multiple of kv_num_heads). All checks run before any launch.
#include "../../include/pa_latent.h"
#include "pa_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

// Device scratch of pa_latent_attention_noalloc: the workspace that entry
// point uses instead of a caller-provided one. Each device the library runs
// on holds its own copy for the life of the process. In host code `scratch`
// names a host-side stand-in, not the device array: its device address comes
// from hipGetSymbolAddress, once per device (static_scratch below).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// kv_num_heads: 0 for the latent layout (one latent head), else the key/value
// heads of the separate layout.
pa_status resolve(const pa_latent_attrs* a, const pa_latent_dims* d, pa_dtype dtype, pa::CallGeom* g,
                  int kv_num_heads = 0) {
  if (!a) return fail(PA_ERR_INVALID_ARGUMENT, "attrs is NULL");
  if (!d) return fail(PA_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_NOT_IMPLEMENTED, "dtype %d: only float16 (10) and bfloat16 (16) are implemented", (int)dtype);
  if (a->num_heads < 1) return fail(PA_ERR_INVALID_ARGUMENT, "num_heads must be >= 1, got %d", a->num_heads);
  const bool sep = kv_num_heads != 0;
  if (sep && (kv_num_heads < 1 || a->num_heads % kv_num_heads != 0))
    return fail(PA_ERR_INVALID_ARGUMENT, "num_heads (%d) must be a multiple of kv_num_heads (%d)", a->num_heads,
                kv_num_heads);
  if (a->head_size < 8 || a->head_size % 8 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "head_size must be a positive multiple of 8, got %d", a->head_size);
  const int hs = a->head_size;
  const int vhs = a->v_head_size == 0 ? hs : a->v_head_size;
  if (vhs < 1) return fail(PA_ERR_INVALID_ARGUMENT, "v_head_size %d must be in 1..=head_size %d", vhs, hs);
  if (sep && (vhs > hs || vhs % 8 != 0))
    return fail(PA_ERR_NOT_IMPLEMENTED, "separate layout: v_head_size %d must be a multiple of 8 and <= head_size %d",
                vhs, hs);
  if (vhs > hs)
    return fail(PA_ERR_INVALID_ARGUMENT, "v_head_size %d must be in 1..=head_size %d", vhs, hs);
  const int bs = a->block_size;
  if (bs < 16 || (bs & (bs - 1)) != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "block_size must be a power of two >= 16, got %d", bs);
  int rd = 0, ro = 0;
  if (a->do_rotary) {
    rd = a->rotary_dim;
    ro = a->rotary_offset;
    if (rd <= 0 || rd % 16 != 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "rotary_dim must be a positive multiple of 16 (cos_cache.shape[1] %% 8 == 0), got %d", rd);
    if (hs % 16 != 0) return fail(PA_ERR_INVALID_ARGUMENT, "head_size must be a multiple of 16 with rotary, got %d", hs);
    if (rd / 2 > hs / 2) return fail(PA_ERR_INVALID_ARGUMENT, "cos_cache.shape[1] %d exceeds head_size / 2", rd / 2);
    if (ro < 0 || ro % 8 != 0) return fail(PA_ERR_INVALID_ARGUMENT, "rotary_offset must be a non-negative multiple of 8, got %d", ro);
    if (ro + rd > hs)
      return fail(PA_ERR_INVALID_ARGUMENT, "rotary_offset %d + rotary_dim %d exceeds head_size %d", ro, rd, hs);
    if (d->rotary_rows < 1) return fail(PA_ERR_INVALID_ARGUMENT, "rotary_rows must be >= 1 with rotary");
  }
  float scale;
  if (a->has_scale) {
    scale = a->scale;
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale must be finite");
  } else if (vhs == hs) {
    scale = 1.0f / std::sqrt((float)hs);
  } else {
    return fail(PA_ERR_INVALID_ARGUMENT, "explicit 'scale' is required when v_head_size (%d) != head_size (%d)", vhs, hs);
  }
  if (std::isnan(a->softcap)) return fail(PA_ERR_INVALID_ARGUMENT, "softcap is NaN");
  if (d->token_count < 0) return fail(PA_ERR_INVALID_ARGUMENT, "token_count must be >= 0");
  if (d->batch < 1) return fail(PA_ERR_INVALID_ARGUMENT, "batch must be >= 1, got %d", d->batch);
  if (d->max_blocks_per_seq < 1) return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq must be >= 1");
  if (d->num_blocks < 1) return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks must be >= 1");
  if (d->token_count * (int64_t)a->num_heads > (int64_t)INT32_MAX / 2)
    return fail(PA_ERR_INVALID_ARGUMENT, "token_count * num_heads exceeds the grid limit");
  if ((int64_t)d->max_blocks_per_seq * bs > (int64_t)INT32_MAX / 2)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq * block_size exceeds the position range");
  if (d->num_blocks * (int64_t)bs > (int64_t)INT32_MAX)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks * block_size exceeds the int32 slot range");
  if (sep && (int64_t)d->batch * kv_num_heads > (int64_t)INT32_MAX / 8)
    return fail(PA_ERR_INVALID_ARGUMENT, "batch * kv_num_heads exceeds the schedule's range");
  if (sep && (int64_t)bs * kv_num_heads * hs * 2 > (int64_t)INT32_MAX / 2)
    return fail(PA_ERR_INVALID_ARGUMENT, "block_size * kv_num_heads * head_size exceeds a cache block's range");
  g->dtype = (int)dtype;
  g->H = a->num_heads;
  g->hs = hs;
  g->vhs = vhs;
  g->bs = bs;
  int l2 = 0;
  while ((1 << l2) < bs) ++l2;
  g->bs_log2 = l2;
  g->do_rotary = a->do_rotary ? 1 : 0;
  g->interleaved = a->rotary_interleaved ? 1 : 0;
  g->rd = rd;
  g->ro = ro;
  g->window = a->local_window_size < 0 ? -1 : a->local_window_size;
  g->softcap = a->softcap > 0.0f ? a->softcap : 0.0f;
  g->scale = scale;
  g->T = d->token_count;
  g->B = d->batch;
  g->MB = d->max_blocks_per_seq;
  g->NB = d->num_blocks;
  g->P = d->rotary_rows;
  g->sep = sep ? 1 : 0;
  g->kvh = sep ? kv_num_heads : 1;
  return PA_OK;
}

pa_status check_ptr(const void* p, const char* name, bool needed) {
  if (!needed) return PA_OK;
  if (!p) return fail(PA_ERR_INVALID_ARGUMENT, "required input '%s' is NULL", name);
  if (!aligned16(p)) return fail(PA_ERR_INVALID_ARGUMENT, "'%s' must be 16-byte aligned", name);
  return PA_OK;
}

pa_status device_error(hipError_t e, const char* what) {
  return fail(PA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Warmed call signatures (docs.rs page, PagedCaptureSignature and the warm
// gate in execute; PR #1978 "Invariants held": capture/replay safe after a
// warmed call). A call made while its stream is being captured into a HIP
// graph must have run eagerly before with the same signature on the same
// device: the first eager call is where the library's one-time host work
// happens (occupancy query, code-object load on the device, the static
// scratch address), none of which may run inside a capture.
enum Phase { kWrite = 0, kAttention = 1, kAttentionNoAlloc = 2, kForward = 3 };

struct Signature {
  int32_t device, phase, dtype, split, kvh;
  pa_latent_attrs a;
  pa_latent_dims d;
};

Signature make_signature(int device, int phase, pa_dtype dtype, int split, const pa_latent_attrs* a,
                         const pa_latent_dims* d, int kvh = 0) {
  Signature s;
  std::memset(&s, 0, sizeof(s));   // padding bytes take part in the comparison
  s.device = device;
  s.phase = phase;
  s.dtype = (int32_t)dtype;
  s.split = split;
  s.kvh = kvh;
  std::memcpy(&s.a, a, sizeof(*a));
  std::memcpy(&s.d, d, sizeof(*d));
  return s;
}

std::mutex g_warm_mu;
std::vector<Signature> g_warm;      // most recent last; bounded
constexpr size_t kMaxWarm = 1024;

bool is_warmed(const Signature& s) {
  std::lock_guard<std::mutex> lk(g_warm_mu);
  for (const auto& w : g_warm)
    if (std::memcmp(&w, &s, sizeof(s)) == 0) return true;
  return false;
}

void mark_warmed(const Signature& s) {
  std::lock_guard<std::mutex> lk(g_warm_mu);
  for (const auto& w : g_warm)
    if (std::memcmp(&w, &s, sizeof(s)) == 0) return;
  if (g_warm.size() >= kMaxWarm) g_warm.erase(g_warm.begin());
  g_warm.push_back(s);
}

// Whether `stream` is being captured; a capture of an unwarmed signature is
// rejected before anything is enqueued.
pa_status capture_gate(void* stream, const Signature& s, bool* capturing) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing((hipStream_t)stream, &cs);
  if (e != hipSuccess) return device_error(e, "hipStreamIsCapturing");
  *capturing = cs != hipStreamCaptureStatusNone;
  if (*capturing && !is_warmed(s))
    return fail(PA_ERR_CAPTURE_NOT_WARMED,
                "stream capture of a call whose signature (dtype, attributes, shapes, device) has not run "
                "eagerly: make the same call once outside the capture first");
  return PA_OK;
}

// Events registered by pa_latent_profile_next for this thread's next attention call.
thread_local hipEvent_t g_prof_ev[2] = {nullptr, nullptr};

pa_status attention_impl(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                         const void* query, const void* key_cache, const void* cos_cache, const void* sin_cache,
                         const int32_t* cumseq, const int32_t* past, const int32_t* block_table, void* output,
                         void* workspace, size_t workspace_bytes, bool split_kv, void* stream,
                         int phase = kAttention, int kvh = 0, const void* value_cache = nullptr,
                         const pa::FusedWrite* fw = nullptr) {
  hipEvent_t ev[2] = {g_prof_ev[0], g_prof_ev[1]};
  g_prof_ev[0] = g_prof_ev[1] = nullptr;
  const bool timed = ev[0] != nullptr && ev[1] != nullptr;
  pa::CallGeom g;
  pa_status st = resolve(attrs, dims, dtype, &g, kvh);
  if (st != PA_OK) return st;
  const bool any = g.T > 0;
  if ((st = check_ptr(query, "query", any)) != PA_OK) return st;
  if ((st = check_ptr(key_cache, "key_cache", any)) != PA_OK) return st;
  if ((st = check_ptr(value_cache, "value_cache", any && g.sep)) != PA_OK) return st;
  if ((st = check_ptr(cumseq, "cumulative_sequence_length", any)) != PA_OK) return st;
  if ((st = check_ptr(past, "past_seqlens", any)) != PA_OK) return st;
  if ((st = check_ptr(block_table, "block_table", any)) != PA_OK) return st;
  if ((st = check_ptr(output, "output", any)) != PA_OK) return st;
  if ((st = check_ptr(cos_cache, "cos_cache", any && g.do_rotary)) != PA_OK) return st;
  if ((st = check_ptr(sin_cache, "sin_cache", any && g.do_rotary)) != PA_OK) return st;
  if (fw) {
    if ((st = check_ptr(fw->key, "key", any)) != PA_OK) return st;
    if ((st = check_ptr(fw->value, "value", any && g.sep)) != PA_OK) return st;
    if ((st = check_ptr(fw->slot_mapping, "slot_mapping", any)) != PA_OK) return st;
  }
  pa::AttnConfig cfg;
  if (!pa::choose_config(g, &cfg))
    return fail(PA_ERR_NOT_IMPLEMENTED, "no attention instance for head_size %d / v_head_size %d (built: %s)", g.hs,
                g.vhs, g.sep ? "separate layout <= 128 / <= 128" : "<= 576 / <= 512");
  if (!any) { g_last_error.clear(); return PA_OK; }
  if (!workspace) return fail(PA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(PA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  int dev = 0, cus = 0, occ = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(e, "hipGetDevice");
  const Signature sig = make_signature(dev, phase, dtype, split_kv ? 1 : 0, attrs, dims, kvh);
  bool capturing = false;
  if ((st = capture_gate(stream, sig, &capturing)) != PA_OK) return st;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return device_error(e, "hipDeviceGetAttribute");
  e = pa::attn_occupancy(g, cfg, dev, &occ);
  if (e != hipSuccess) return device_error(e, "occupancy query");
  const pa::WsLayout ws = pa::plan_workspace(g, cfg, cus, occ, split_kv);
  if (workspace_bytes < ws.total)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes %zu < required %zu", workspace_bytes, ws.total);
  e = pa::launch_attention(g, cfg, ws, split_kv, query, key_cache, value_cache, cos_cache, sin_cache, cumseq, past,
                           block_table, output, workspace, (hipStream_t)stream, timed ? ev : nullptr, fw);
  if (e != hipSuccess) return device_error(e, "attention launch");
  if (!capturing) mark_warmed(sig);
  g_last_error.clear();
  return PA_OK;
}

// Device address of `scratch` on the current device `dev`, looked up on the
// first call on that device (with it current) and kept per device.
pa_status static_scratch(int dev, void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) { *ptr = it->second; return PA_OK; }
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return device_error(e, "hipGetSymbolAddress(scratch)");
  if (!p) return fail(PA_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
  addr[dev] = p;
  *ptr = p;
  return PA_OK;
}

pa_status write_impl(const pa_latent_attrs* attrs, int kvh, const pa_latent_dims* dims, pa_dtype dtype,
                     const void* key, const void* value, const void* cos_cache, const void* sin_cache,
                     const int32_t* slot_mapping, const int32_t* cumseq, const int32_t* past, void* key_cache,
                     void* value_cache, void* stream) {
  pa::CallGeom g;
  pa_status st = resolve(attrs, dims, dtype, &g, kvh);
  if (st != PA_OK) return st;
  const bool any = g.T > 0;
  if ((st = check_ptr(key, "key", any)) != PA_OK) return st;
  if ((st = check_ptr(value, "value", any && g.sep)) != PA_OK) return st;
  if ((st = check_ptr(slot_mapping, "slot_mapping", any)) != PA_OK) return st;
  if ((st = check_ptr(cumseq, "cumulative_sequence_length", any)) != PA_OK) return st;
  if ((st = check_ptr(past, "past_seqlens", any)) != PA_OK) return st;
  if ((st = check_ptr(key_cache, "key_cache", any)) != PA_OK) return st;
  if ((st = check_ptr(value_cache, "value_cache", any && g.sep)) != PA_OK) return st;
  if ((st = check_ptr(cos_cache, "cos_cache", any && g.do_rotary)) != PA_OK) return st;
  if ((st = check_ptr(sin_cache, "sin_cache", any && g.do_rotary)) != PA_OK) return st;
  if (!any) { g_last_error.clear(); return PA_OK; }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(e, "hipGetDevice");
  const Signature sig = make_signature(dev, kWrite, dtype, 0, attrs, dims, kvh);
  bool capturing = false;
  if ((st = capture_gate(stream, sig, &capturing)) != PA_OK) return st;
  e = pa::launch_write(g, key, value, cos_cache, sin_cache, slot_mapping, cumseq, past, key_cache, value_cache,
                       (hipStream_t)stream);
  if (e != hipSuccess) return device_error(e, "write launch");
  if (!capturing) mark_warmed(sig);
  g_last_error.clear();
  return PA_OK;
}

pa_status workspace_impl(const pa_latent_attrs* attrs, int kvh, const pa_latent_dims* dims, pa_dtype dtype,
                         int device, size_t* bytes) {
  if (!bytes) return fail(PA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = 0;
  pa::CallGeom g;
  pa_status st = resolve(attrs, dims, dtype, &g, kvh);
  if (st != PA_OK) return st;
  pa::AttnConfig cfg;
  if (!pa::choose_config(g, &cfg))
    return fail(PA_ERR_NOT_IMPLEMENTED, "no attention instance for head_size %d / v_head_size %d", g.hs, g.vhs);
  int cus = 0, occ = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return device_error(e, "hipDeviceGetAttribute");
  e = pa::attn_occupancy(g, cfg, device, &occ);
  if (e != hipSuccess) return device_error(e, "occupancy query");
  // Size for the larger of the two partitions so either entry point fits.
  const pa::WsLayout a = pa::plan_workspace(g, cfg, cus, occ, true);
  const pa::WsLayout b = pa::plan_workspace(g, cfg, cus, occ, false);
  *bytes = a.total > b.total ? a.total : b.total;
  g_last_error.clear();
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_latent_write(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                          const void* key, const void* cos_cache, const void* sin_cache,
                          const int32_t* slot_mapping, const int32_t* cumulative_sequence_length,
                          const int32_t* past_seqlens, void* key_cache, void* stream) {
  return write_impl(attrs, 0, dims, dtype, key, nullptr, cos_cache, sin_cache, slot_mapping,
                    cumulative_sequence_length, past_seqlens, key_cache, nullptr, stream);
}

pa_status pa_latent_workspace_size(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                                   int device, size_t* bytes) {
  return workspace_impl(attrs, 0, dims, dtype, device, bytes);
}

pa_status pa_latent_attention(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                              const void* query, const void* key_cache, const void* cos_cache,
                              const void* sin_cache, const int32_t* cumulative_sequence_length,
                              const int32_t* past_seqlens, const int32_t* block_table, void* output,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(attrs, dims, dtype, query, key_cache, cos_cache, sin_cache, cumulative_sequence_length,
                        past_seqlens, block_table, output, workspace, workspace_bytes, true, stream);
}

pa_status pa_latent_forward(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                            const void* query, const void* key, const void* cos_cache, const void* sin_cache,
                            const int32_t* slot_mapping, const int32_t* cumulative_sequence_length,
                            const int32_t* past_seqlens, const int32_t* block_table, void* key_cache, void* output,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const pa::FusedWrite fw{key, slot_mapping, key_cache, nullptr, nullptr};
  return attention_impl(attrs, dims, dtype, query, key_cache, cos_cache, sin_cache, cumulative_sequence_length,
                        past_seqlens, block_table, output, workspace, workspace_bytes, true, stream, kForward, 0,
                        nullptr, &fw);
}

pa_status pa_latent_attention_splits(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                                     const void* query, const void* key_cache, const void* cos_cache,
                                     const void* sin_cache, const int32_t* cumulative_sequence_length,
                                     const int32_t* past_seqlens, const int32_t* block_table, void* output,
                                     void* workspace, size_t workspace_bytes, int32_t split_kv, void* stream) {
  return attention_impl(attrs, dims, dtype, query, key_cache, cos_cache, sin_cache, cumulative_sequence_length,
                        past_seqlens, block_table, output, workspace, workspace_bytes, split_kv != 0, stream);
}

pa_status pa_latent_attention_noalloc(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                                      const void* query, const void* key_cache, const void* cos_cache,
                                      const void* sin_cache, const int32_t* cumulative_sequence_length,
                                      const int32_t* past_seqlens, const int32_t* block_table, void* output,
                                      void* stream) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_prof_ev[0] = g_prof_ev[1] = nullptr;
    return device_error(e, "hipGetDevice");
  }
  void* ws = nullptr;
  size_t need = 0;
  pa_status st = PA_OK;
  if (attrs && dims && dims->token_count > 0) {
    // The first call on a device looks up the scratch address: not inside a capture.
    bool capturing = false;
    st = capture_gate(stream, make_signature(dev, kAttentionNoAlloc, dtype, 1, attrs, dims), &capturing);
  }
  if (st == PA_OK) st = static_scratch(dev, &ws);
  if (st == PA_OK) st = pa_latent_workspace_size(attrs, dims, dtype, dev, &need);
  if (st == PA_OK && need > kStaticScratchBytes)
    st = fail(PA_ERR_WORKSPACE_TOO_SMALL,
              "pa_latent_attention_noalloc: this call needs %zu bytes of scratch; the library's static scratch "
              "holds %zu (use pa_latent_attention with a caller workspace)",
              need, kStaticScratchBytes);
  if (st != PA_OK) {
    g_prof_ev[0] = g_prof_ev[1] = nullptr;   // the registration is consumed by this call
    return st;
  }
  return attention_impl(attrs, dims, dtype, query, key_cache, cos_cache, sin_cache, cumulative_sequence_length,
                        past_seqlens, block_table, output, ws, kStaticScratchBytes, true, stream, kAttentionNoAlloc);
}

pa_status pa_separate_write(const pa_latent_attrs* attrs, int32_t kv_num_heads, const pa_latent_dims* dims,
                            pa_dtype dtype, const void* key, const void* value, const void* cos_cache,
                            const void* sin_cache, const int32_t* slot_mapping,
                            const int32_t* cumulative_sequence_length, const int32_t* past_seqlens, void* key_cache,
                            void* value_cache, void* stream) {
  if (kv_num_heads < 1) return fail(PA_ERR_INVALID_ARGUMENT, "kv_num_heads must be >= 1, got %d", kv_num_heads);
  return write_impl(attrs, kv_num_heads, dims, dtype, key, value, cos_cache, sin_cache, slot_mapping,
                    cumulative_sequence_length, past_seqlens, key_cache, value_cache, stream);
}

pa_status pa_separate_workspace_size(const pa_latent_attrs* attrs, int32_t kv_num_heads, const pa_latent_dims* dims,
                                     pa_dtype dtype, int device, size_t* bytes) {
  if (bytes) *bytes = 0;
  if (kv_num_heads < 1) return fail(PA_ERR_INVALID_ARGUMENT, "kv_num_heads must be >= 1, got %d", kv_num_heads);
  return workspace_impl(attrs, kv_num_heads, dims, dtype, device, bytes);
}

pa_status pa_separate_attention(const pa_latent_attrs* attrs, int32_t kv_num_heads, const pa_latent_dims* dims,
                                pa_dtype dtype, const void* query, const void* key_cache, const void* value_cache,
                                const void* cos_cache, const void* sin_cache,
                                const int32_t* cumulative_sequence_length, const int32_t* past_seqlens,
                                const int32_t* block_table, void* output, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (kv_num_heads < 1) {
    g_prof_ev[0] = g_prof_ev[1] = nullptr;
    return fail(PA_ERR_INVALID_ARGUMENT, "kv_num_heads must be >= 1, got %d", kv_num_heads);
  }
  return attention_impl(attrs, dims, dtype, query, key_cache, cos_cache, sin_cache, cumulative_sequence_length,
                        past_seqlens, block_table, output, workspace, workspace_bytes, true, stream, kAttention,
                        kv_num_heads, value_cache);
}

pa_status pa_separate_forward(const pa_latent_attrs* attrs, int32_t kv_num_heads, const pa_latent_dims* dims,
                              pa_dtype dtype, const void* query, const void* key, const void* value,
                              const void* cos_cache, const void* sin_cache, const int32_t* slot_mapping,
                              const int32_t* cumulative_sequence_length, const int32_t* past_seqlens,
                              const int32_t* block_table, void* key_cache, void* value_cache, void* output,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_num_heads < 1) {
    g_prof_ev[0] = g_prof_ev[1] = nullptr;
    return fail(PA_ERR_INVALID_ARGUMENT, "kv_num_heads must be >= 1, got %d", kv_num_heads);
  }
  const pa::FusedWrite fw{key, slot_mapping, key_cache, value, value_cache};
  return attention_impl(attrs, dims, dtype, query, key_cache, cos_cache, sin_cache, cumulative_sequence_length,
                        past_seqlens, block_table, output, workspace, workspace_bytes, true, stream, kForward,
                        kv_num_heads, value_cache, &fw);
}

pa_status pa_latent_capture_ready(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                                  int device, int32_t* write_ready, int32_t* attention_ready) {
  if (!attrs || !dims || !write_ready || !attention_ready)
    return fail(PA_ERR_INVALID_ARGUMENT, "NULL argument to pa_latent_capture_ready");
  *write_ready = is_warmed(make_signature(device, kWrite, dtype, 0, attrs, dims)) ? 1 : 0;
  *attention_ready = is_warmed(make_signature(device, kAttention, dtype, 1, attrs, dims)) ? 1 : 0;
  g_last_error.clear();
  return PA_OK;
}

pa_status pa_latent_profile_next(void* before, void* after) {
  g_prof_ev[0] = (hipEvent_t)before;
  g_prof_ev[1] = (hipEvent_t)after;
  g_last_error.clear();
  return PA_OK;
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int32_t pa_latent_abi_version(void) { return PA_LATENT_ABI_VERSION; }

}  // extern "C"
