// Host side of the multi-layer decode step (include/longflow_stack.h):
// argument checks, workspace layout, the per-layer launch sequence and its
// capture into a HIP graph.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <vector>

#include "launch.h"
#include "stack_launch.h"
#include "layout.h"
#include "longflow.h"
#include "longflow_stack.h"

namespace {

constexpr int kMaxStackBatch = 256;  // two 128-row blocks of the projection kernel

struct StackLayout {
  size_t dec, q, k, v, o, x0, x1, scores, rope, part, total;
};

StackLayout stack_layout(int B, int H, int Hq, int Hkv, int d, int S, size_t dec_bytes) {
  StackLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = lf::align_up(off + bytes, 256);
    return at;
  };
  w.dec = take(dec_bytes);  // first: lf_read_device_status reads its status word
  w.q = take((size_t)B * Hq * d * 2);
  w.k = take((size_t)B * Hkv * d * 2);
  w.v = take((size_t)B * Hkv * d * 2);
  w.o = take((size_t)B * Hq * d * 2);
  w.x0 = take((size_t)B * H * 2);
  w.x1 = take((size_t)B * H * 2);
  w.scores = take((size_t)B * Hkv * S * 4);
  w.rope = take((size_t)B * (d / 2) * 8);
  const size_t p1 = lf::gemm_partial_bytes(B, (Hq + 2 * Hkv) * d, H);
  const size_t p2 = lf::gemm_partial_bytes(B, H, Hq * d);
  w.part = take(p1 > p2 ? p1 : p2);
  w.total = off;
  return w;
}

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_stack_shape(int L, int B, int H, int Hq, int Hkv, int d, int S) {
  if (L < 1 || B < 1 || B > kMaxStackBatch || H < 256 || H % 256 != 0) return LF_E_SHAPE;
  int rc = lf_check_shape(B, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if ((Hq * d) % 256 != 0) return LF_E_SHAPE;  // K of the output projection
  return LF_OK;
}

struct StackArgs {
  int L, B, H, Hq, Hkv, d, S;
  float scale, rope_base;
  const void* x_in;
  void* x_out;
  int32_t* pos;
  int advance_pos;
  const void* const* w_qkv;
  const void* const* w_o;
  void* const* k_cache;
  void* const* v_cache;
  const uint8_t* const* mask;
  int32_t* const* slot;
  float* const* scores;
  void* workspace;
  size_t workspace_bytes;
  int nsplit;
};

int resolve_nsplit(StackArgs& a) {
  if (a.nsplit < 0) return LF_E_NSPLIT;
  if (a.nsplit == 0) {
    int cus = 0;
    int rc = lf_device_num_cus(&cus);
    if (rc != LF_OK) return rc;
    rc = lf_plan_nsplit(a.B, a.Hq, a.Hkv, a.d, a.S, cus, &a.nsplit);
    if (rc != LF_OK) return rc;
  }
  return LF_OK;
}

int validate_stack(const StackArgs& a) {
  int rc = check_stack_shape(a.L, a.B, a.H, a.Hq, a.Hkv, a.d, a.S);
  if (rc != LF_OK) return rc;
  if (!std::isfinite(a.scale) || !std::isfinite(a.rope_base) || a.rope_base <= 0.f) return LF_E_VALUE;
  if (!a.x_in || !a.x_out || !a.pos || !a.w_qkv || !a.w_o || !a.k_cache || !a.v_cache || !a.mask ||
      !a.slot || !a.workspace)
    return LF_E_NULL;
  size_t dec_bytes = 0;
  rc = lf_workspace_size(a.B, a.Hq, a.Hkv, a.d, a.S, a.nsplit, &dec_bytes);
  if (rc != LF_OK) return rc;
  const int gp = lf::padded_group(a.Hq / a.Hkv);
  int len, eff;
  lf::split_geometry(a.S, a.nsplit, &len, &eff);
  if (len > lf::max_split_len(a.d, gp)) return LF_E_NSPLIT;
  const StackLayout wl = stack_layout(a.B, a.H, a.Hq, a.Hkv, a.d, a.S, dec_bytes);

  const size_t B = a.B, H = a.H, Hq = a.Hq, Hkv = a.Hkv, d = a.d, S = a.S;
  struct Buf {
    const void* p;
    size_t n;
    bool written;
  };
  std::vector<Buf> bufs;
  bufs.push_back({a.x_in, B * H * 2, false});
  bufs.push_back({a.x_out, B * H * 2, true});
  bufs.push_back({a.pos, B * 4, a.advance_pos != 0});
  bufs.push_back({a.workspace, wl.total, true});
  for (int l = 0; l < a.L; ++l) {
    if (!a.w_qkv[l] || !a.w_o[l] || !a.k_cache[l] || !a.v_cache[l] || !a.mask[l] || !a.slot[l])
      return LF_E_NULL;
    if (misaligned(a.w_qkv[l], 16) || misaligned(a.w_o[l], 16) || misaligned(a.k_cache[l], 16) ||
        misaligned(a.v_cache[l], 16) || misaligned(a.slot[l], 4) ||
        (a.scores && a.scores[l] && misaligned(a.scores[l], 4)))
      return LF_E_ALIGN;
    bufs.push_back({a.w_qkv[l], (Hq + 2 * Hkv) * d * H * 2, false});
    bufs.push_back({a.w_o[l], H * Hq * d * 2, false});
    bufs.push_back({a.k_cache[l], B * Hkv * S * d * 2, true});
    bufs.push_back({a.v_cache[l], B * Hkv * S * d * 2, true});
    bufs.push_back({a.mask[l], B * S, false});
    bufs.push_back({a.slot[l], B * Hkv * 4, true});
    if (a.scores && a.scores[l]) bufs.push_back({a.scores[l], B * Hkv * S * 4, true});
  }
  if (misaligned(a.x_in, 16) || misaligned(a.x_out, 16) || misaligned(a.pos, 4) ||
      misaligned(a.workspace, 256))
    return LF_E_ALIGN;
  for (size_t i = 0; i < bufs.size(); ++i)
    for (size_t j = i + 1; j < bufs.size(); ++j)
      if ((bufs[i].written || bufs[j].written) && overlaps(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
        return LF_E_ALIAS;
  if (a.workspace_bytes < wl.total) return LF_E_WORKSPACE;
  return LF_OK;
}

// Every launch of one step, in order, on `s` (valid arguments assumed).
int enqueue_stack(const StackArgs& a, hipStream_t s) {
  size_t dec_bytes = 0;
  lf_workspace_size(a.B, a.Hq, a.Hkv, a.d, a.S, a.nsplit, &dec_bytes);
  const StackLayout wl = stack_layout(a.B, a.H, a.Hq, a.Hkv, a.d, a.S, dec_bytes);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  uint16_t* q = reinterpret_cast<uint16_t*>(ws + wl.q);
  uint16_t* kn = reinterpret_cast<uint16_t*>(ws + wl.k);
  uint16_t* vn = reinterpret_cast<uint16_t*>(ws + wl.v);
  uint16_t* o = reinterpret_cast<uint16_t*>(ws + wl.o);
  uint16_t* xb[2] = {reinterpret_cast<uint16_t*>(ws + wl.x0), reinterpret_cast<uint16_t*>(ws + wl.x1)};
  float* ws_scores = reinterpret_cast<float*>(ws + wl.scores);
  float* part = reinterpret_cast<float*>(ws + wl.part);
  float2* rope = reinterpret_cast<float2*>(ws + wl.rope);
  const int nq = (a.Hq + 2 * a.Hkv) * a.d;
  const lf::RopeParams rp{a.pos, rope, q, kn, vn, a.B, a.Hq, a.Hkv, a.d, std::log2((double)a.rope_base)};

  // The positions hold for every layer of the step: one rotation table.
  if (lf::launch_rope_table(rp, s) != hipSuccess) return LF_E_HIP;
  for (int l = 0; l < a.L; ++l) {
    const uint16_t* xin = l == 0 ? static_cast<const uint16_t*>(a.x_in) : xb[(l - 1) & 1];
    uint16_t* xout = l == a.L - 1 ? static_cast<uint16_t*>(a.x_out) : xb[l & 1];
    lf::GemmParams g1{xin, static_cast<const uint16_t*>(a.w_qkv[l]), nullptr, nullptr, part, a.B, nq, a.H, 0, 0};
    if (lf::launch_gemm(g1, s, &rp) != hipSuccess) return LF_E_HIP;
    float* sc = (a.scores && a.scores[l]) ? a.scores[l] : ws_scores;
    int rc = lf::enqueue_decode_step(a.B, a.Hq, a.Hkv, a.d, a.S, a.scale, q, a.k_cache[l], a.v_cache[l],
                                     a.mask[l], nullptr, kn, vn, a.slot[l], o, sc, a.slot[l],
                                     ws + wl.dec, a.nsplit, LF_SPLIT_AUTO, s);
    if (rc != LF_OK) return rc;
    lf::GemmParams g2{o, static_cast<const uint16_t*>(a.w_o[l]), xin, xout, part, a.B, a.H, a.Hq * a.d, 0, 0};
    if (lf::launch_gemm(g2, s) != hipSuccess) return LF_E_HIP;
  }
  if (a.advance_pos && lf::launch_advance_pos(a.pos, a.B, s) != hipSuccess) return LF_E_HIP;
  return LF_OK;
}

}  // namespace

extern "C" {

int lf_stack_workspace_size(int L, int B, int H, int Hq, int Hkv, int d, int S, int nsplit,
                            size_t* bytes) {
  if (!bytes) return LF_E_NULL;
  int rc = check_stack_shape(L, B, H, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  size_t dec = 0;
  rc = lf_workspace_size(B, Hq, Hkv, d, S, nsplit, &dec);
  if (rc != LF_OK) return rc;
  *bytes = stack_layout(B, H, Hq, Hkv, d, S, dec).total;
  return LF_OK;
}

int lf_stack_workspace_offsets(int B, int H, int Hq, int Hkv, int d, int S, int nsplit,
                               size_t* offsets) {
  if (!offsets) return LF_E_NULL;
  int rc = check_stack_shape(1, B, H, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  size_t dec = 0;
  rc = lf_workspace_size(B, Hq, Hkv, d, S, nsplit < 1 ? -1 : nsplit, &dec);
  if (rc != LF_OK) return rc;
  const StackLayout w = stack_layout(B, H, Hq, Hkv, d, S, dec);
  offsets[0] = w.q;
  offsets[1] = w.k;
  offsets[2] = w.v;
  offsets[3] = w.o;
  return LF_OK;
}

int longflow_stack_step(int L, int B, int H, int Hq, int Hkv, int d, int S, float scale,
                        float rope_base, const void* x_in, void* x_out, int32_t* pos,
                        int advance_pos, const void* const* w_qkv, const void* const* w_o,
                        void* const* k_cache, void* const* v_cache, const uint8_t* const* mask,
                        int32_t* const* slot, float* const* scores, void* workspace,
                        size_t workspace_bytes, int nsplit, void* stream) {
  StackArgs a{L, B, H, Hq, Hkv, d, S, scale, rope_base, x_in, x_out, pos, advance_pos, w_qkv,
              w_o, k_cache, v_cache, mask, slot, scores, workspace, workspace_bytes, nsplit};
  int rc = check_stack_shape(L, B, H, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if ((rc = resolve_nsplit(a)) != LF_OK) return rc;
  if ((rc = validate_stack(a)) != LF_OK) return rc;
  return enqueue_stack(a, static_cast<hipStream_t>(stream));
}

int lf_stack_graph_create(int L, int B, int H, int Hq, int Hkv, int d, int S, float scale,
                          float rope_base, const void* x_in, void* x_out, int32_t* pos,
                          int advance_pos, const void* const* w_qkv, const void* const* w_o,
                          void* const* k_cache, void* const* v_cache, const uint8_t* const* mask,
                          int32_t* const* slot, float* const* scores, void* workspace,
                          size_t workspace_bytes, int nsplit, void** graph) {
  if (!graph) return LF_E_NULL;
  *graph = nullptr;
  StackArgs a{L, B, H, Hq, Hkv, d, S, scale, rope_base, x_in, x_out, pos, advance_pos, w_qkv,
              w_o, k_cache, v_cache, mask, slot, scores, workspace, workspace_bytes, nsplit};
  int rc = check_stack_shape(L, B, H, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if ((rc = resolve_nsplit(a)) != LF_OK) return rc;
  if ((rc = validate_stack(a)) != LF_OK) return rc;

  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return LF_E_HIP;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return LF_E_HIP;
  }
  rc = enqueue_stack(a, cs);
  hipGraph_t g = nullptr;
  const hipError_t end = hipStreamEndCapture(cs, &g);
  (void)hipStreamDestroy(cs);
  if (rc != LF_OK || end != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    return rc != LF_OK ? rc : LF_E_HIP;
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t inst = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (inst != hipSuccess || !exec) return LF_E_HIP;
  *graph = exec;
  return LF_OK;
}

int lf_graph_launch(void* graph, void* stream) {
  if (!graph) return LF_E_NULL;
  return hipGraphLaunch(static_cast<hipGraphExec_t>(graph), static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? LF_OK
             : LF_E_HIP;
}

int lf_graph_destroy(void* graph) {
  if (!graph) return LF_E_NULL;
  return hipGraphExecDestroy(static_cast<hipGraphExec_t>(graph)) == hipSuccess ? LF_OK : LF_E_HIP;
}

}  // extern "C"
