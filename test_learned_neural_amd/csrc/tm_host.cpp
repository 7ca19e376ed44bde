// Host side of the C ABI declared in include/titans_mem.h: argument
// validation (before anything is enqueued), kernel selection and launch.
#include <string.h>

#include "tm_internal.h"

namespace {

using titans::Shape;

int build_shape(const titans_mem_desc* desc, Shape* s) {
  if (!desc) return TM_ERR_INVALID;
  if (desc->abi_version != TITANS_MEM_ABI_VERSION) return TM_ERR_INVALID;
  if (desc->B <= 0 || desc->H <= 0 || desc->N < 0 || desc->d <= 0 || desc->n_layers <= 0)
    return TM_ERR_INVALID;
  if (desc->n_layers >= 2 && desc->hidden <= 0) return TM_ERR_INVALID;
  if (desc->activation != TM_ACT_SILU) return TM_ERR_INVALID;
  if (desc->io_dtype != TM_IO_F32 && desc->io_dtype != TM_IO_BF16) return TM_ERR_INVALID;
  if (desc->read_mode != TM_READ_AFTER_WRITE && desc->read_mode != TM_READ_CHUNK_START)
    return TM_ERR_INVALID;
  if (desc->flags & ~(TM_FLAG_FORCE_GENERIC | TM_FLAG_CHUNK_GATES | TM_FLAG_NO_WAIT)) return TM_ERR_INVALID;
  if (desc->n_layers > titans::kMaxLayers) return TM_ERR_UNSUPPORTED;
  const int64_t streams = (int64_t)desc->B * desc->H;
  if (streams > (int64_t)1 << 30) return TM_ERR_UNSUPPORTED;
  s->streams = (int)streams;
  s->N = desc->N;
  s->d = desc->d;
  s->hidden = desc->n_layers >= 2 ? desc->hidden : 0;
  s->L = desc->n_layers;
  s->io = desc->io_dtype;
  s->read_mode = desc->read_mode;
  s->chunk_gates = (desc->flags & TM_FLAG_CHUNK_GATES) ? 1 : 0;
  s->flags = desc->flags;
  s->widths[0] = desc->d;
  for (int l = 1; l < s->L; ++l) s->widths[l] = desc->hidden;
  s->widths[s->L] = desc->d;
  s->P = 0;
  s->maxw = 0;
  for (int l = 0; l <= s->L; ++l)
    if (s->widths[l] > s->maxw) s->maxw = s->widths[l];
  for (int l = 1; l <= s->L; ++l) {
    s->off[l] = s->P;
    s->P += (int64_t)s->widths[l] * s->widths[l - 1];
  }
  return TM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  const char* lo;
  int64_t bytes;
  bool writes;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.lo || !b.lo || a.bytes <= 0 || b.bytes <= 0) return false;
  return a.lo < b.lo + b.bytes && b.lo < a.lo + a.bytes;
}

int select_path(const titans_mem_desc* desc, const Shape& s, int chunk) {
  if (chunk <= 0) return TM_ERR_INVALID;
  if (!(desc->flags & TM_FLAG_FORCE_GENERIC) && titans::mlp2_supported(s, chunk))
    return TM_PATH_MLP2_D64_H256;
  if (!(desc->flags & TM_FLAG_FORCE_GENERIC) && titans::deep_supported(s, chunk)) return TM_PATH_DEEP_BF16;
  if (chunk > titans::kMaxChunkGeneric || s.maxw > titans::kMaxWidthGeneric) return TM_ERR_UNSUPPORTED;
  return TM_PATH_GENERIC_F32;
}

int64_t workspace_for(const Shape& s, int path, int chunk) {
  if (path == TM_PATH_MLP2_D64_H256) return titans::mlp2_ws_bytes(s, chunk);
  if (path == TM_PATH_DEEP_BF16) return titans::deep_ws_bytes(s, chunk);
  return titans::generic_forward_ws_floats_per_stream(s, chunk) * (int64_t)sizeof(float) * s.streams;
}

}  // namespace

extern "C" {

int32_t titans_mem_abi_version(void) { return TITANS_MEM_ABI_VERSION; }

int64_t titans_mem_param_count(const titans_mem_desc* desc) {
  Shape s;
  int rc = build_shape(desc, &s);
  return rc ? rc : s.P;
}

int32_t titans_mem_select_path(const titans_mem_desc* desc, int32_t chunk) {
  Shape s;
  int rc = build_shape(desc, &s);
  if (rc) return rc;
  return select_path(desc, s, chunk);
}

int64_t titans_mem_workspace_bytes(const titans_mem_desc* desc, int32_t chunk) {
  Shape s;
  int rc = build_shape(desc, &s);
  if (rc) return rc;
  int path = select_path(desc, s, chunk);
  if (path < 0) return path;
  return workspace_for(s, path, chunk);
}

}  // extern "C"

namespace {

// Validation shared by titans_mem_forward and titans_mem_forward_noalloc:
// pointers, path, workspace size (has_ws: the caller passes one) and
// aliasing, all on the host.  Fills s and path.
int check_forward(const titans_mem_desc* desc, const void* k, const void* v, const void* q, const float* alpha,
                  const float* eta, const float* theta, const float* W_in, const float* S_in, int32_t chunk,
                  const void* y_out, const float* W_out, const float* S_out, const void* workspace,
                  int64_t workspace_bytes, bool has_ws, Shape* sp, int* path_out) {
  Shape& s = *sp;
  int rc = build_shape(desc, &s);
  if (rc) return rc;
  if (chunk <= 0) return TM_ERR_INVALID;
  const bool has_tokens = s.N > 0;
  const void* token_ptrs[] = {k, v, q, alpha, eta, theta, y_out};
  for (const void* p : token_ptrs) {
    if (has_tokens && !p) return TM_ERR_INVALID;
    if (p && !aligned16(p)) return TM_ERR_INVALID;
  }
  const void* state_ptrs[] = {W_in, S_in, W_out, S_out};
  for (const void* p : state_ptrs)
    if (!p || !aligned16(p)) return TM_ERR_INVALID;
  if (workspace && !aligned16(workspace)) return TM_ERR_INVALID;
  int path = select_path(desc, s, chunk);
  if (path < 0) return path;
  const int64_t need = has_ws ? workspace_for(s, path, chunk) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need)) return TM_ERR_WORKSPACE;

  const int64_t esz = s.io == TM_IO_BF16 ? 2 : 4;
  const int64_t tok_bytes = (int64_t)s.streams * s.N * s.d * esz;
  const int64_t gate_rows = s.chunk_gates ? ((int64_t)s.N + chunk - 1) / chunk : s.N;
  const int64_t gate_bytes = (int64_t)s.streams * gate_rows * 4;
  const int64_t state_bytes = (int64_t)s.streams * s.P * 4;
  const Range ranges[] = {
      {(const char*)k, tok_bytes, false},          {(const char*)v, tok_bytes, false},
      {(const char*)q, tok_bytes, false},          {(const char*)alpha, gate_bytes, false},
      {(const char*)eta, gate_bytes, false},       {(const char*)theta, gate_bytes, false},
      {(const char*)W_in, state_bytes, false},     {(const char*)S_in, state_bytes, false},
      {(const char*)y_out, tok_bytes, true},       {(const char*)W_out, state_bytes, true},
      {(const char*)S_out, state_bytes, true},     {(const char*)workspace, need, true},
  };
  const int nr = sizeof(ranges) / sizeof(ranges[0]);
  for (int i = 0; i < nr; ++i) {
    for (int j = i + 1; j < nr; ++j) {
      if (!ranges[i].writes && !ranges[j].writes) continue;
      if (!overlap(ranges[i], ranges[j])) continue;
      // exact in-place state update is the one allowed overlap
      const bool w_inplace = i == 6 && j == 9 && (const void*)W_in == (const void*)W_out;
      const bool s_inplace = i == 7 && j == 10 && (const void*)S_in == (const void*)S_out;
      if (w_inplace || s_inplace) continue;
      return TM_ERR_ALIAS;
    }
  }
  *path_out = path;
  return TM_OK;
}

}  // namespace

extern "C" {

int titans_mem_forward(const titans_mem_desc* desc, const void* k, const void* v, const void* q,
                       const float* alpha, const float* eta, const float* theta,
                       const float* W_in, const float* S_in, int32_t chunk, void* y_out,
                       float* W_out, float* S_out, void* workspace, int64_t workspace_bytes,
                       void* stream) {
  Shape s;
  int path = 0;
  int rc = check_forward(desc, k, v, q, alpha, eta, theta, W_in, S_in, chunk, y_out, W_out, S_out, workspace,
                         workspace_bytes, true, &s, &path);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipError_t err;
  if (path == TM_PATH_MLP2_D64_H256)
    err = titans::launch_mlp2(s, chunk, k, v, q, alpha, eta, theta, W_in, S_in, y_out, W_out, S_out,
                          workspace, st);
  else if (path == TM_PATH_DEEP_BF16)
    err = titans::launch_deep(s, chunk, k, v, q, alpha, eta, theta, W_in, S_in, y_out, W_out, S_out, workspace, st);
  else
    err = titans::launch_generic(s, chunk, k, v, q, alpha, eta, theta, W_in, S_in, y_out, W_out,
                             S_out, (float*)workspace, st);
  return err == hipSuccess ? TM_OK : TM_ERR_HIP;
}

int titans_mem_forward_noalloc(const titans_mem_desc* desc, const void* k, const void* v, const void* q,
                               const float* alpha, const float* eta, const float* theta, const float* W_in,
                               const float* S_in, int32_t chunk, void* y_out, float* W_out, float* S_out,
                               void* stream) {
  Shape s;
  int path = 0;
  int rc = check_forward(desc, k, v, q, alpha, eta, theta, W_in, S_in, chunk, y_out, W_out, S_out, nullptr, 0,
                         false, &s, &path);
  if (rc) return rc;
  if (path != TM_PATH_MLP2_D64_H256) return TM_ERR_UNSUPPORTED;
  if (titans::mlp2_ws_bytes(s, chunk) > titans::mlp2_scratch_bytes()) return TM_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (titans::mlp2_scratch(&scratch, true) != hipSuccess || !scratch) return TM_ERR_HIP;
  hipError_t err = titans::launch_mlp2(s, chunk, k, v, q, alpha, eta, theta, W_in, S_in, y_out, W_out, S_out,
                                       scratch, (hipStream_t)stream);
  return err == hipSuccess ? TM_OK : TM_ERR_HIP;
}

int titans_mem_workspace_status(const titans_mem_desc* desc, int32_t chunk, const void* workspace,
                                int64_t workspace_bytes, void* stream) {
  Shape s;
  int rc = build_shape(desc, &s);
  if (rc) return rc;
  const int path = select_path(desc, s, chunk);
  if (path < 0) return path;
  const hipStream_t st = (hipStream_t)stream;
  if (path != TM_PATH_MLP2_D64_H256)
    return hipStreamSynchronize(st) == hipSuccess ? TM_OK : TM_ERR_HIP;
  if (workspace && !aligned16(workspace)) return TM_ERR_INVALID;
  if (!workspace) {
    // the allocation-free variant's scratch on this device (never used: nothing to report)
    void* scratch = nullptr;
    if (titans::mlp2_scratch(&scratch, false) != hipSuccess) return TM_ERR_HIP;
    if (!scratch) return hipStreamSynchronize(st) == hipSuccess ? TM_OK : TM_ERR_HIP;
    workspace = scratch;
    workspace_bytes = titans::mlp2_scratch_bytes();
  }
  const int64_t need = workspace_for(s, path, chunk);
  if (workspace_bytes < need) return TM_ERR_WORKSPACE;
  unsigned word = 0;
  if (hipMemcpyAsync(&word, (const char*)workspace + titans::mlp2_status_offset(s), sizeof(word),
                     hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return TM_ERR_HIP;
  return word ? TM_ERR_GAVE_UP : TM_OK;
}

int titans_mem_retrieve(const titans_mem_desc* desc, const void* q, const float* W, void* y_out,
                        void* stream) {
  Shape s;
  int rc = build_shape(desc, &s);
  if (rc) return rc;
  if (s.N > 0 && (!q || !y_out)) return TM_ERR_INVALID;
  if (!W || !aligned16(W) || (q && !aligned16(q)) || (y_out && !aligned16(y_out)))
    return TM_ERR_INVALID;
  const bool mfma = !(desc->flags & TM_FLAG_FORCE_GENERIC) && titans::retrieve_mlp2_supported(s);
  if (!mfma && s.maxw > titans::kMaxWidthRetrieve) return TM_ERR_UNSUPPORTED;
  const int64_t esz = s.io == TM_IO_BF16 ? 2 : 4;
  const int64_t tok_bytes = (int64_t)s.streams * s.N * s.d * esz;
  const Range yr = {(const char*)y_out, tok_bytes, true};
  if (overlap(yr, Range{(const char*)q, tok_bytes, false}) ||
      overlap(yr, Range{(const char*)W, (int64_t)s.streams * s.P * 4, false}))
    return TM_ERR_ALIAS;
  if (s.N == 0) return TM_OK;
  hipError_t err = mfma ? titans::launch_retrieve_mlp2(s, q, W, y_out, (hipStream_t)stream)
                        : titans::launch_retrieve_generic(s, q, W, y_out, (hipStream_t)stream);
  return err == hipSuccess ? TM_OK : TM_ERR_HIP;
}

int64_t titans_mem_backward_workspace_bytes(const titans_mem_desc* desc, int32_t chunk) {
  Shape s;
  int rc = build_shape(desc, &s);
  if (rc) return rc;
  if (chunk <= 0) return TM_ERR_INVALID;
  if (!titans::backward_supported(s, chunk)) return TM_ERR_UNSUPPORTED;
  return titans::backward_ws_floats_per_stream(s, chunk) * (int64_t)sizeof(float) * s.streams;
}

int titans_mem_backward(const titans_mem_desc* desc, const void* k, const void* v, const void* q,
                        const float* alpha, const float* eta, const float* theta, const float* W_in,
                        const float* S_in, int32_t chunk, const float* dy, const float* dW_out,
                        const float* dS_out, float* dk, float* dv, float* dq, float* dalpha, float* deta,
                        float* dtheta, float* dW_in, float* dS_in, void* workspace, int64_t workspace_bytes,
                        void* stream) {
  Shape s;
  int rc = build_shape(desc, &s);
  if (rc) return rc;
  if (chunk <= 0) return TM_ERR_INVALID;
  const void* required[] = {k, v, q, alpha, eta, theta, W_in, S_in, dk, dv, dq, dalpha, deta, dtheta, dW_in, dS_in};
  for (const void* p : required)
    if (!p || !aligned16(p)) return TM_ERR_INVALID;
  const void* optional[] = {dy, dW_out, dS_out, workspace};
  for (const void* p : optional)
    if (p && !aligned16(p)) return TM_ERR_INVALID;
  if (!titans::backward_supported(s, chunk)) return TM_ERR_UNSUPPORTED;
  const int64_t need = titans::backward_ws_floats_per_stream(s, chunk) * (int64_t)sizeof(float) * s.streams;
  if (!workspace || workspace_bytes < need) return TM_ERR_WORKSPACE;
  const int64_t esz = s.io == TM_IO_BF16 ? 2 : 4;
  const int64_t tok = (int64_t)s.streams * s.N * s.d;
  const int64_t gate_rows = s.chunk_gates ? ((int64_t)s.N + chunk - 1) / chunk : s.N;
  const int64_t gates = (int64_t)s.streams * gate_rows * 4;
  const int64_t state = (int64_t)s.streams * s.P * 4;
  const Range ranges[] = {
      {(const char*)k, tok * esz, false},   {(const char*)v, tok * esz, false},
      {(const char*)q, tok * esz, false},   {(const char*)alpha, gates, false},
      {(const char*)eta, gates, false},     {(const char*)theta, gates, false},
      {(const char*)W_in, state, false},    {(const char*)S_in, state, false},
      {(const char*)dy, tok * 4, false},    {(const char*)dW_out, state, false},
      {(const char*)dS_out, state, false},  {(const char*)dk, tok * 4, true},
      {(const char*)dv, tok * 4, true},     {(const char*)dq, tok * 4, true},
      {(const char*)dalpha, gates, true},   {(const char*)deta, gates, true},
      {(const char*)dtheta, gates, true},   {(const char*)dW_in, state, true},
      {(const char*)dS_in, state, true},    {(const char*)workspace, need, true},
  };
  const int nr = sizeof(ranges) / sizeof(ranges[0]);
  for (int i = 0; i < nr; ++i)
    for (int j = i + 1; j < nr; ++j)
      if ((ranges[i].writes || ranges[j].writes) && overlap(ranges[i], ranges[j])) return TM_ERR_ALIAS;
  hipError_t err = titans::launch_backward(s, chunk, k, v, q, alpha, eta, theta, W_in, S_in, dy, dW_out, dS_out,
                                           dk, dv, dq, dalpha, deta, dtheta, dW_in, dS_in, (float*)workspace,
                                           (hipStream_t)stream);
  return err == hipSuccess ? TM_OK : TM_ERR_HIP;
}

int titans_mem_input(const titans_input_desc* desc, const void* x, const void* w_proj, const float* conv_w,
                     const void* w_gate, const float* b_gate, float alpha_scale, float eta_scale,
                     float theta_scale, void* k_out, void* v_out, void* q_out, float* alpha_out,
                     float* eta_out, float* theta_out, void* stream) {
  if (!desc || desc->abi_version != TITANS_MEM_ABI_VERSION) return TM_ERR_INVALID;
  if (desc->B <= 0 || desc->N < 0 || desc->D <= 0 || desc->H <= 0 || desc->d <= 0 || desc->conv_width <= 0 ||
      desc->flags != 0)
    return TM_ERR_INVALID;
  if (!titans::input_supported(desc->D, desc->H, desc->d, desc->conv_width)) return TM_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, w_proj, conv_w, w_gate, b_gate, k_out, v_out, q_out, alpha_out, eta_out, theta_out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return TM_ERR_INVALID;
  const int64_t R = (int64_t)desc->B * desc->N;
  const int64_t C = (int64_t)desc->H * desc->d;
  if (titans::input_grid(R, desc->D, desc->H, desc->d, desc->conv_width) >= ((int64_t)1 << 31))
    return TM_ERR_UNSUPPORTED;
  const int64_t tok = R * C * 2, gate = R * desc->H * 4;
  const Range ranges[] = {
      {(const char*)x, R * desc->D * 2, false},
      {(const char*)w_proj, 3 * C * desc->D * 2, false},
      {(const char*)conv_w, 3 * C * desc->conv_width * 4, false},
      {(const char*)w_gate, (int64_t)3 * desc->H * desc->D * 2, false},
      {(const char*)b_gate, (int64_t)3 * desc->H * 4, false},
      {(const char*)k_out, tok, true},     {(const char*)v_out, tok, true},
      {(const char*)q_out, tok, true},     {(const char*)alpha_out, gate, true},
      {(const char*)eta_out, gate, true},  {(const char*)theta_out, gate, true},
  };
  const int nr = sizeof(ranges) / sizeof(ranges[0]);
  for (int i = 0; i < nr; ++i)
    for (int j = i + 1; j < nr; ++j)
      if ((ranges[i].writes || ranges[j].writes) && overlap(ranges[i], ranges[j])) return TM_ERR_ALIAS;
  if (R == 0) return TM_OK;
  const float scale[3] = {alpha_scale, eta_scale, theta_scale};
  void* const kvq[3] = {k_out, v_out, q_out};
  float* const gates[3] = {alpha_out, eta_out, theta_out};
  hipError_t err = titans::launch_input(desc->B, desc->N, desc->D, desc->H, desc->d, desc->conv_width, x, w_proj,
                                        conv_w, w_gate, b_gate, scale, kvq, gates, (hipStream_t)stream);
  return err == hipSuccess ? TM_OK : TM_ERR_HIP;
}

const char* titans_mem_status_string(int status) {
  switch (status) {
    case TM_OK: return "ok";
    case TM_ERR_INVALID: return "invalid argument";
    case TM_ERR_UNSUPPORTED: return "unsupported shape, dtype or flag combination";
    case TM_ERR_WORKSPACE: return "workspace too small";
    case TM_ERR_ALIAS: return "illegal buffer overlap";
    case TM_ERR_HIP: return "HIP launch error";
    case TM_ERR_GAVE_UP: return "paired workgroups gave up waiting for each other; outputs are NaN";
    default: return "unknown status";
  }
}

}  // extern "C"
