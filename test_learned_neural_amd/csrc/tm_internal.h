// Internal declarations shared by the host layer and the kernel files of
// libtitans_mem.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "titans_mem.h"

namespace titans {

constexpr int kMaxLayers = 8;        // generic path
constexpr int kMaxChunkGeneric = 4096;
constexpr int kMaxWidthGeneric = 8192;
constexpr int kRetrieveTile = 8;     // tokens per block in titans_mem_retrieve
constexpr int kMaxWidthRetrieve = 1024;

struct Shape {
  int streams, N, d, hidden, L, io, read_mode;
  int chunk_gates;   // gates given per chunk (TM_FLAG_CHUNK_GATES)
  unsigned flags;    // the desc's TM_FLAG_* bits
  int widths[kMaxLayers + 1];
  int64_t off[kMaxLayers + 1];
  int64_t P;
  int maxw;
};

// Workspace floats per stream of the generic kernel for chunk b (one region).
int64_t generic_ws_floats_per_stream(const Shape& s, int b);
// Workspace floats per stream of launch_generic (the forward call).
int64_t generic_forward_ws_floats_per_stream(const Shape& s, int chunk);

// The library's second stream on a device and the events that order it
// against the caller's stream: created on first use (default priority) and
// kept until the process ends.  side_stream() returns the current device's
// with `lock` held, which serialises the calls that enqueue on it (each
// call records every event before waiting on it).
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, prod[2] = {nullptr, nullptr}, cons[2] = {nullptr, nullptr};
};
hipError_t side_stream(int dev, SideStream** out, std::unique_lock<std::mutex>& lock);
// Makes `stream` wait for everything enqueued so far on the side stream.
// Every launcher calls it on each return path after its first enqueue on the
// side stream (errors included), so that work the caller enqueues on
// `stream` afterwards, such as freeing buffers, never overtakes it; returns
// `err` when that is an error, else the join's own status.
hipError_t join_side(SideStream* x, hipStream_t stream, hipError_t err);

hipError_t launch_generic(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                          const float* alpha, const float* eta, const float* theta,
                          const float* W_in, const float* S_in, void* y, float* W_out,
                          float* S_out, float* ws, hipStream_t stream);

hipError_t launch_retrieve_generic(const Shape& s, const void* q, const float* W, void* y,
                                   hipStream_t stream);

// The linear memory (L = 1, d <= 64 and a multiple of 4, chunk <= 64) on one
// workgroup per stream with the state and the chunk in LDS; part of the
// generic path (fp32 arithmetic, no workspace).
bool linear_supported(const Shape& s, int chunk);
hipError_t launch_linear(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                         const float* alpha, const float* eta, const float* theta, const float* W_in,
                         const float* S_in, void* y, float* W_out, float* S_out, hipStream_t stream);

// Specialised 2-layer d=64 hidden=256 MFMA kernel (chunk <= 64, bf16 io).
bool mlp2_supported(const Shape& s, int chunk);
int64_t mlp2_ws_bytes(const Shape& s, int chunk);
// byte offset of the kernel's status word in its workspace (1 = a pair gave up)
int64_t mlp2_status_offset(const Shape& s);
// The allocation-free variant's scratch: a file-scope device array of
// mlp2_scratch_bytes() bytes in tm_mlp2_group.hip.  mlp2_scratch gives its device
// address on the current device, looked up there on the first call with
// lookup = true (nullptr while it never was).
int64_t mlp2_scratch_bytes();
hipError_t mlp2_scratch(void** out, bool lookup);
hipError_t launch_mlp2(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                       const float* alpha, const float* eta, const float* theta,
                       const float* W_in, const float* S_in, void* y, float* W_out,
                       float* S_out, void* ws, hipStream_t stream);

// Deep memories on the matrix cores: L >= 2, widths multiples of 64, bf16 io,
// chunk <= 256; one launch per step of a chunk over all streams.
bool deep_supported(const Shape& s, int chunk);
int64_t deep_ws_bytes(const Shape& s, int chunk);
hipError_t launch_deep(const Shape& s, int chunk, const void* k, const void* v, const void* q, const float* alpha,
                       const float* eta, const float* theta, const float* W_in, const float* S_in, void* y,
                       float* W_out, float* S_out, void* ws, hipStream_t stream);

// Retrieval at a fixed state on the matrix cores (2-layer, d=64, hidden=256, bf16).
bool retrieve_mlp2_supported(const Shape& s);
hipError_t launch_retrieve_mlp2(const Shape& s, const void* q, const float* W, void* y, hipStream_t stream);

// The generic kernel as a state sweep only (no retrieval), writing (W, S) at
// every chunk start to ckpt; W, S and ckpt are strided per stream.  The last
// chunk is not folded: W, S end at its start state.
hipError_t launch_generic_checkpoints(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                                      const float* alpha, const float* eta, const float* theta, const float* W_in,
                                      const float* S_in, float* W, float* S, int64_t state_stride, float* ckpt,
                                      int64_t ckpt_stride, float* ws, int64_t ws_stride, hipStream_t stream);

// Backward pass through the memory (generic fp32, one workgroup per stream).
constexpr int kMaxWidthBackward = 1024;
bool backward_supported(const Shape& s, int chunk);
int64_t backward_ws_floats_per_stream(const Shape& s, int chunk);
hipError_t launch_backward(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                           const float* alpha, const float* eta, const float* theta, const float* W_in,
                           const float* S_in, const float* dy, const float* dW_out, const float* dS_out, float* dk,
                           float* dv, float* dq, float* dalpha, float* deta, float* dtheta, float* dW_in,
                           float* dS_in, float* ws, hipStream_t stream);

// Input side (x -> k, v, q and the gates): bf16 MFMA GEMM with a fused
// convolution / SiLU / l2-norm / sigmoid epilogue.
bool input_supported(int D, int H, int d, int w);
int64_t input_grid(int64_t R, int D, int H, int d, int w);
hipError_t launch_input(int B, int N, int D, int H, int d, int w, const void* x, const void* w_proj,
                        const float* conv_w, const void* w_gate, const float* b_gate, const float scale[3],
                        void* const kvq[3], float* const gates[3], hipStream_t stream);

}  // namespace titans
