// C-ABI entry points of libhils: argument validation, workspace sizing and
// kernel dispatch. Every check happens before anything is enqueued.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "hils.h"
#include "hils_internal.h"

namespace {
// Static scratch of hils_score_topk_noalloc: one copy per GPU, held until the
// process ends. Host code never uses the name below as an address; it uses the
// device address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = (size_t)16 << 20;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of the current device's scratch, looked up once per device.
hils_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return HILS_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return HILS_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HILS_OK;
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hils_status resolve(const hils_dims* in, hils::Dims* out) {
  if (in == nullptr || out == nullptr) return HILS_ERR_INVALID_ARG;
  const hils_dims& d = *in;
  if (d.window < 0) return HILS_ERR_INVALID_ARG;
  if (d.select_mode != HILS_SELECT_PER_HEAD && d.select_mode != HILS_SELECT_GROUP_MAX)
    return HILS_ERR_INVALID_ARG;
  if (d.B < 1 || d.Tq < 0 || d.Tkv < 1 || d.H < 1 || d.Hkv < 1 || d.H % d.Hkv != 0)
    return HILS_ERR_INVALID_ARG;
  if (d.dtype != HILS_F32 && d.dtype != HILS_BF16) return HILS_ERR_INVALID_ARG;
  if (d.S < 1 || d.d < 1 || d.K < 1) return HILS_ERR_INVALID_ARG;
  if (d.S != hils::kChunk || (d.d != 64 && d.d != 128) || d.K > hils::kMaxSel) return HILS_ERR_UNSUPPORTED;
  if (d.window % d.S != 0 || d.window > hils::kMaxWinChunks * d.S) return HILS_ERR_UNSUPPORTED;
  if (d.q_pos0 < 0 || d.q_pos0 + d.Tq > d.Tkv) return HILS_ERR_INVALID_ARG;
  if (d.Tkv_cap < 0 || d.NC_cap < 0) return HILS_ERR_INVALID_ARG;
  const int Tcap = d.Tkv_cap ? d.Tkv_cap : d.Tkv;
  if (Tcap < d.Tkv) return HILS_ERR_INVALID_ARG;
  const int NCcap = d.NC_cap ? d.NC_cap : Tcap / d.S;
  if (NCcap < d.Tkv / d.S) return HILS_ERR_INVALID_ARG;
  if (!std::isfinite(d.scale) || d.scale < 0.0f) return HILS_ERR_INVALID_ARG;
  out->B = d.B;
  out->Tq = d.Tq;
  out->Tkv = d.Tkv;
  out->Tcap = Tcap;
  out->NCcap = NCcap;
  out->H = d.H;
  out->Hkv = d.Hkv;
  out->G = d.H / d.Hkv;
  out->d = d.d;
  out->S = d.S;
  out->K = d.K;
  out->bf16 = d.dtype == HILS_BF16;
  out->q_pos0 = d.q_pos0;
  out->scale = d.scale != 0.0f ? d.scale : 1.0f / std::sqrt((float)d.d);
  out->group_sel = d.select_mode == HILS_SELECT_GROUP_MAX;
  out->window = d.window;
  if (out->group_sel && ((out->G & (out->G - 1)) != 0 || out->G > 64)) return HILS_ERR_UNSUPPORTED;
  return HILS_OK;
}

// K and V of a decode cache may live in pinned host memory (hipHostMalloc): the
// kernels then read through its device mapping, so only the chunks a call
// touches cross the host link. Device memory passes unchanged; memory no
// kernel can read (pageable host memory) is rejected.
hils_status kv_view(const void* p, const void** out) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return HILS_ERR_INVALID_ARG;
  }
  if (a.type == hipMemoryTypeHost) {
    if (a.devicePointer == nullptr) return HILS_ERR_INVALID_ARG;
    *out = a.devicePointer;
  } else if (a.type == hipMemoryTypeDevice) {
    *out = p;
  } else {
    return HILS_ERR_INVALID_ARG;  // unregistered (pageable) or other memory kinds
  }
  return HILS_OK;
}

hils_status backward_shape_ok(const hils::Dims& dm) {
  if (dm.q_pos0 != 0 || dm.Tq != dm.Tkv || dm.Tkv % dm.S != 0) return HILS_ERR_UNSUPPORTED;
  return HILS_OK;
}

hils_status from_hip(hipError_t e) { return e == hipSuccess ? HILS_OK : HILS_ERR_HIP; }

// A decode step of few rows runs as split scoring, then a slot kernel that
// merges the split lists itself, then the combine: the lists and the slot
// partials are live together, lists first. A step of many rows (sequences
// decoding together) runs as split scoring, then one workgroup per row that
// merges once, attends every slot and fuses them in LDS. Otherwise the step is
// the two calls one after the other on the stream, which share the larger of
// their workspaces.
enum DecodePlan { kDecodeCalls = 0, kDecodeMerged = 1, kDecodeRow = 2 };
// rows from which one workgroup per row pays: on 128K caches, 128 rows (8
// sequences of 16 heads) 33.7 against 35.0 us per step with the merge, slot and
// combine launches, 256 rows 48.0 against 51.0 us
constexpr long long kDecodeRowMin = 128;
DecodePlan decode_plan(const hils::Dims& dm, int* ns, int* km) {
  *ns = 0;
  if (!hils::attend_is_decode(dm)) return kDecodeCalls;
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  // every slot's workgroup repeats its row's merge: worth it while the slots
  // fill the chip about once (a K = 16 step of 16 heads: 272 workgroups); with
  // more slots the separate merge launch costs less than the repeated merges
  const long long slots = rows * (dm.K + dm.nlocal_max());
  if (slots > 384 && rows < kDecodeRowMin) return kDecodeCalls;
  *ns = hils::decode_lists_plan(dm, km);
  if (*ns == 0) return kDecodeCalls;
  if (slots <= 384) return kDecodeMerged;
  return hils::decode_row_applies(dm, *ns, *km) ? kDecodeRow : kDecodeCalls;
}
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_ws(const hils::Dims& dm) {
  int km = 0, ns = 0;
  const DecodePlan pl = decode_plan(dm, &ns, &km);
  if (pl == kDecodeMerged)
    return align256(hils::decode_lists_ws_bytes(dm, ns)) + hils::attend_ws_bytes(dm);
  const size_t a = hils::score_topk_ws_bytes(dm), b = hils::attend_ws_bytes(dm);
  const size_t calls = a > b ? a : b;
  // the row plan needs only the lists; it also covers the two calls, which the
  // same shape takes at positions with no candidates, so a workspace sized for
  // any position serves every position of the shape
  if (pl == kDecodeRow) return std::max(hils::decode_lists_ws_bytes(dm, ns), calls);
  return calls;
}

hils_status check_ws(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return HILS_OK;
  if (ws_bytes < need) return HILS_ERR_WORKSPACE;
  if (!aligned16(ws)) return HILS_ERR_INVALID_ARG;
  return HILS_OK;
}

}  // namespace

extern "C" {

hils_status hils_workspace_size(const hils_dims* dims, int op, size_t* bytes) {
  hils::Dims dm;
  if (bytes == nullptr) return HILS_ERR_INVALID_ARG;
  hils_status st = resolve(dims, &dm);
  if (st != HILS_OK) return st;
  switch (op) {
    case HILS_OP_SUMMARIZE: *bytes = 0; return HILS_OK;
    case HILS_OP_SCORE_TOPK: *bytes = hils::score_topk_ws_bytes(dm); return HILS_OK;
    case HILS_OP_ATTEND_FUSE: *bytes = hils::attend_ws_bytes(dm); return HILS_OK;
    case HILS_OP_DECODE: *bytes = decode_ws(dm); return HILS_OK;
    case HILS_OP_BACKWARD:
      st = backward_shape_ok(dm);
      if (st != HILS_OK) return st;
      *bytes = hils::backward_ws_bytes(dm);
      return HILS_OK;
    default: return HILS_ERR_INVALID_ARG;
  }
}

hils_status hils_summarize(const hils_dims* dims, const void* K, const void* Ql, int32_t c_begin,
                           int32_t c_end, float* ksum, float* ent, float* lse_l, void* ws,
                           size_t ws_bytes, hils_stream stream) {
  (void)ws;
  (void)ws_bytes;
  hils::Dims dm;
  hils_status st = resolve(dims, &dm);
  if (st != HILS_OK) return st;
  if (c_begin < 0 || c_end < c_begin || c_end > dm.Tkv / dm.S || c_end > dm.NCcap)
    return HILS_ERR_INVALID_ARG;
  if (c_end == c_begin) return HILS_OK;
  if (!aligned16(K) || !aligned16(Ql) || !aligned16(ksum) || !aligned16(ent)) return HILS_ERR_INVALID_ARG;
  if (lse_l != nullptr && !aligned16(lse_l)) return HILS_ERR_INVALID_ARG;
  const void* Kd = nullptr;
  st = kv_view(K, &Kd);
  if (st != HILS_OK) return st;
  return from_hip(hils::launch_summarize(dm, Kd, Ql, c_begin, c_end, ksum, ent, lse_l,
                                         reinterpret_cast<hipStream_t>(stream)));
}

hils_status hils_score_topk(const hils_dims* dims, const void* Q, const float* ksum,
                            const float* ent, int32_t* idx, float* score, void* ws,
                            size_t ws_bytes, hils_stream stream) {
  hils::Dims dm;
  hils_status st = resolve(dims, &dm);
  if (st != HILS_OK) return st;
  if (dm.Tq == 0) return HILS_OK;
  if (!aligned16(Q) || !aligned16(ksum) || !aligned16(ent) || !aligned16(idx) || !aligned16(score))
    return HILS_ERR_INVALID_ARG;
  st = check_ws(hils::score_topk_ws_bytes(dm), ws, ws_bytes);
  if (st != HILS_OK) return st;
  return from_hip(hils::launch_score_topk(dm, Q, ksum, ent, idx, score, ws,
                                          reinterpret_cast<hipStream_t>(stream)));
}

hils_status hils_score_topk_noalloc(const hils_dims* dims, const void* Q, const float* ksum,
                                    const float* ent, int32_t* idx, float* score,
                                    hils_stream stream) {
  hils::Dims dm;
  hils_status st = resolve(dims, &dm);
  if (st != HILS_OK) return st;
  if (dm.Tq == 0) return HILS_OK;
  if (!aligned16(Q) || !aligned16(ksum) || !aligned16(ent) || !aligned16(idx) || !aligned16(score))
    return HILS_ERR_INVALID_ARG;
  const size_t need = hils::score_topk_ws_bytes(dm);
  if (need > kScratchBytes) return HILS_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && (st = scratch_of_current_device(&ws)) != HILS_OK) return st;
  return from_hip(hils::launch_score_topk(dm, Q, ksum, ent, idx, score, ws,
                                          reinterpret_cast<hipStream_t>(stream)));
}

hils_status hils_attend_fuse(const hils_dims* dims, const void* Q, const void* K, const void* V,
                             const int32_t* idx, const float* score, void* O, float* lse_own,
                             float* lse_tot, void* ws, size_t ws_bytes, hils_stream stream) {
  hils::Dims dm;
  hils_status st = resolve(dims, &dm);
  if (st != HILS_OK) return st;
  if (dm.Tq == 0) return HILS_OK;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(idx) || !aligned16(score) ||
      !aligned16(O))
    return HILS_ERR_INVALID_ARG;
  if ((lse_own != nullptr && !aligned16(lse_own)) || (lse_tot != nullptr && !aligned16(lse_tot)))
    return HILS_ERR_INVALID_ARG;
  st = check_ws(hils::attend_ws_bytes(dm), ws, ws_bytes);
  if (st != HILS_OK) return st;
  const void *Kd = nullptr, *Vd = nullptr;
  if ((st = kv_view(K, &Kd)) != HILS_OK || (st = kv_view(V, &Vd)) != HILS_OK) return st;
  return from_hip(hils::launch_attend_fuse(dm, Q, Kd, Vd, idx, score, O, lse_own, lse_tot, ws,
                                           reinterpret_cast<hipStream_t>(stream)));
}

hils_status hils_decode(const hils_dims* dims, const void* Q, const void* K, const void* V,
                        const float* ksum, const float* ent, int32_t* idx, float* score, void* O,
                        float* lse_own, float* lse_tot, void* ws, size_t ws_bytes,
                        hils_stream stream) {
  hils::Dims dm;
  hils_status st = resolve(dims, &dm);
  if (st != HILS_OK) return st;
  if (dm.Tq == 0) return HILS_OK;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(ksum) || !aligned16(ent) ||
      !aligned16(idx) || !aligned16(score) || !aligned16(O))
    return HILS_ERR_INVALID_ARG;
  if ((lse_own != nullptr && !aligned16(lse_own)) || (lse_tot != nullptr && !aligned16(lse_tot)))
    return HILS_ERR_INVALID_ARG;
  st = check_ws(decode_ws(dm), ws, ws_bytes);
  if (st != HILS_OK) return st;
  const void *Kd = nullptr, *Vd = nullptr;
  if ((st = kv_view(K, &Kd)) != HILS_OK || (st = kv_view(V, &Vd)) != HILS_OK) return st;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  int km = 0, ns = 0;
  const DecodePlan pl = decode_plan(dm, &ns, &km);
  if (pl != kDecodeCalls) {
    const long long nl = (long long)dm.B * dm.Tq * dm.H * ns * dm.K;
    float* ws_s = reinterpret_cast<float*>(ws);
    int* ws_i = reinterpret_cast<int*>(ws_s + nl);
    hipError_t e = hils::launch_decode_lists(dm, Q, ksum, ent, ws_s, ws_i, ns, hs);
    if (e != hipSuccess) return HILS_ERR_HIP;
    if (pl == kDecodeRow)
      return from_hip(hils::launch_decode_row(dm, Q, Kd, Vd, ws_s, ws_i, ns, km, idx, score, O,
                                              lse_own, lse_tot, hs));
    void* ws_a = reinterpret_cast<char*>(ws) + align256(hils::decode_lists_ws_bytes(dm, ns));
    return from_hip(hils::launch_decode_merged(dm, Q, Kd, Vd, ws_s, ws_i, ns, km, idx, score, O,
                                               lse_own, lse_tot, ws_a, hs));
  }
  hipError_t err = hils::launch_score_topk(dm, Q, ksum, ent, idx, score, ws, hs);
  if (err != hipSuccess)
    return HILS_ERR_HIP;
  return from_hip(hils::launch_attend_fuse(dm, Q, Kd, Vd, idx, score, O, lse_own, lse_tot, ws, hs));
}

hils_status hils_backward(const hils_dims* dims, const void* Q, const void* K, const void* V,
                          const void* Ql, const float* ksum, const float* ent,
                          const float* lse_l, const int32_t* idx, const float* score,
                          const float* lse_tot, const void* O, const void* dO, void* dQ,
                          void* dK, void* dV, void* dQl, const void* Qs, void* dQs, void* ws,
                          size_t ws_bytes, hils_stream stream) {
  hils::Dims dm;
  hils_status st = resolve(dims, &dm);
  if (st != HILS_OK) return st;
  st = backward_shape_ok(dm);
  if (st != HILS_OK) return st;
  const void* in[] = {Q, K, V, Ql, ksum, ent, lse_l, idx, score, lse_tot, O, dO, dQ, dK, dV, dQl};
  for (const void* p : in)
    if (!aligned16(p)) return HILS_ERR_INVALID_ARG;
  if ((Qs == nullptr) != (dQs == nullptr)) return HILS_ERR_INVALID_ARG;
  if (Qs != nullptr && (!aligned16(Qs) || !aligned16(dQs))) return HILS_ERR_INVALID_ARG;
  st = check_ws(hils::backward_ws_bytes(dm), ws, ws_bytes);
  if (st != HILS_OK) return st;
  return from_hip(hils::launch_backward(dm, Q, K, V, Ql, ksum, ent, lse_l, idx, score, lse_tot, O,
                                        dO, dQ, dK, dV, dQl, Qs, dQs, ws,
                                        reinterpret_cast<hipStream_t>(stream)));
}

const char* hils_status_string(hils_status status) {
  switch (status) {
    case HILS_OK: return "HILS_OK";
    case HILS_ERR_INVALID_ARG: return "HILS_ERR_INVALID_ARG: null, misaligned or inconsistent argument";
    case HILS_ERR_UNSUPPORTED: return "HILS_ERR_UNSUPPORTED: shape outside S=64, d in {64,128}, K<=64";
    case HILS_ERR_WORKSPACE: return "HILS_ERR_WORKSPACE: workspace smaller than hils_workspace_size";
    case HILS_ERR_HIP: return "HILS_ERR_HIP: kernel launch failed";
    case HILS_ERR_SCRATCH:
      return "HILS_ERR_SCRATCH: the call needs more scratch than the library's static 16 MiB";
    default: return "unknown hils_status";
  }
}

int32_t hils_version(void) { return 100; }

}  // extern "C"
