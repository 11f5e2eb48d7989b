// Decode-step graphs: the step's KV store and paged decode (one kernel, as
// pa_paged_attn_decode_store runs them), captured once per batch bucket (1,
// 2, 4, ... max_batch) as HIP graphs and replayed with one launch ("Nano-vLLM
// System Architecture Analysis", section 2 "CUDA Graphs"; "Differences from
// Normal nanoGPT Inference", item 4). A step of n
// sequences runs the smallest bucket that holds it; the rows between n and the
// bucket are made inert first (slot -1 stores nothing, context 0 writes no
// output), by a small kernel launched outside the graph on the caller's
// stream before every replay; the same kernel writes the replay's fresh
// piece-counter tag into the workspace header, where the captured decode
// reads it (a captured launch keeps its capture-time arguments). Nothing
// inside the graphs clears memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "paged_attn.h"
#include "pa_launch.h"

namespace {

constexpr int32_t kMaxGraphBatch = 512;

__global__ void make_rows_inert(int32_t* slot_mapping, int32_t* context_lens, int32_t from, int32_t to,
                                uint64_t* epoch_word, uint64_t tag) {
  const int32_t t = static_cast<int32_t>(blockIdx.x * blockDim.x + threadIdx.x);
  if (t == 0 && epoch_word != nullptr) __hip_atomic_store(epoch_word, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int32_t i = from + t;
  if (i < to) {
    slot_mapping[i] = -1;
    context_lens[i] = 0;
  }
}

}  // namespace

struct pa_decode_graphs {
  pa_decode_graph_buffers bufs;
  int32_t max_batch = 0;
  std::vector<int32_t> buckets;
  std::vector<hipGraphExec_t> execs;
  std::vector<hipGraph_t> graphs;

  ~pa_decode_graphs() {
    for (hipGraphExec_t e : execs)
      if (e) (void)hipGraphExecDestroy(e);
    for (hipGraph_t g : graphs)
      if (g) (void)hipGraphDestroy(g);
  }
};

extern "C" {

pa_status pa_decode_graphs_create(const pa_decode_graph_buffers* bufs, int32_t max_batch, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, float scale, pa_dtype dtype,
                                  pa_decode_graphs** out) {
  if (out == nullptr) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (bufs == nullptr || max_batch <= 0 || max_batch > kMaxGraphBatch || max_blocks_per_seq <= 0 ||
      block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (bufs->out == nullptr || bufs->q == nullptr || bufs->k_new == nullptr || bufs->v_new == nullptr ||
      bufs->slot_mapping == nullptr || bufs->block_tables == nullptr || bufs->context_lens == nullptr)
    return PA_ERR_INVALID_ARG;
  const int64_t max_ctx64 = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  if (max_ctx64 >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  const int32_t max_ctx = static_cast<int32_t>(max_ctx64);
  // Validate every argument once, as the largest bucket's calls will see
  // them, before any HIP call (a zero-token store and a zero-sequence decode
  // validate without launching).
  pa_status st = pa_kv_store(bufs->k_cache, bufs->v_cache, bufs->k_new, bufs->v_new, bufs->slot_mapping, 0,
                             num_kv_heads, head_dim, block_size, num_blocks, dtype, nullptr);
  if (st != PA_OK) return st;
  st = pa_paged_attn_decode(bufs->out, bufs->q, bufs->k_cache, bufs->v_cache, bufs->block_tables,
                            bufs->context_lens, 0, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                            max_blocks_per_seq, max_ctx, scale, dtype, bufs->workspace, bufs->workspace_bytes,
                            nullptr);
  if (st != PA_OK) return st;
  if (pa_decode_workspace_bytes(max_batch, num_q_heads, head_dim, 0, max_ctx) > bufs->workspace_bytes)
    return PA_ERR_WORKSPACE;

  pa_decode_graphs* g = new (std::nothrow) pa_decode_graphs();
  if (g == nullptr) return PA_ERR_INVALID_ARG;
  g->bufs = *bufs;
  g->max_batch = max_batch;
  for (int32_t b = 1; b < max_batch; b *= 2) g->buckets.push_back(b);
  g->buckets.push_back(max_batch);

  // The decode launcher sizes its grid from a device query it caches; make
  // that query now, outside any capture.
  if (pa_decode_num_workgroups(max_batch, num_q_heads, num_kv_heads, head_dim, max_ctx, dtype) <= 0) {
    delete g;
    return PA_ERR_INVALID_ARG;
  }
  hipStream_t cap;
  if (hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess) {
    delete g;
    return PA_ERR_HIP;
  }
  st = PA_OK;
  for (int32_t b : g->buckets) {
    if (hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      st = PA_ERR_HIP;
      break;
    }
    // one kernel node: the store of the new rows fused with the decode
    const pa_status s2 = pa::decode_store_for_graph(
        bufs->out, bufs->q, bufs->k_cache, bufs->v_cache, bufs->k_new, bufs->v_new, bufs->slot_mapping,
        bufs->block_tables, bufs->context_lens, b, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
        max_blocks_per_seq, max_ctx, scale, dtype, bufs->workspace, bufs->workspace_bytes, cap);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(cap, &graph);  // always leave capture mode
    if (s2 != PA_OK || e != hipSuccess || graph == nullptr) {
      if (graph) (void)hipGraphDestroy(graph);
      st = s2 != PA_OK ? s2 : PA_ERR_HIP;
      break;
    }
    g->graphs.push_back(graph);
    hipGraphExec_t exec = nullptr;
    if (hipGraphInstantiateWithFlags(&exec, graph, 0) != hipSuccess) {
      st = PA_ERR_HIP;
      break;
    }
    g->execs.push_back(exec);
  }
  (void)hipStreamDestroy(cap);
  (void)hipGetLastError();
  if (st != PA_OK) {
    delete g;
    return st;
  }
  *out = g;
  return PA_OK;
}

int32_t pa_decode_graphs_bucket(const pa_decode_graphs* g, int32_t num_seqs) {
  if (g == nullptr || num_seqs <= 0) return 0;
  for (int32_t b : g->buckets)
    if (b >= num_seqs) return b;
  return 0;
}

pa_status pa_decode_graphs_launch(pa_decode_graphs* g, int32_t num_seqs, pa_stream_t stream) {
  if (g == nullptr || num_seqs < 0 || num_seqs > g->max_batch) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  size_t k = 0;
  while (g->buckets[k] < num_seqs) ++k;
  const int32_t bucket = g->buckets[k];
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // every replay: the padding rows (if any) and the replay's counter tag
  const int32_t n = bucket - num_seqs;
  uint64_t* epoch_word =
      g->bufs.workspace ? reinterpret_cast<uint64_t*>(static_cast<char*>(g->bufs.workspace) + pa::kWorkspaceEpochOff)
                        : nullptr;
  make_rows_inert<<<dim3(static_cast<uint32_t>(n > 0 ? (n + 255) / 256 : 1)), dim3(256), 0, s>>>(
      g->bufs.slot_mapping, g->bufs.context_lens, num_seqs, bucket, epoch_word, pa::next_epoch_tag());
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  return hipGraphLaunch(g->execs[k], s) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

void pa_decode_graphs_destroy(pa_decode_graphs* g) { delete g; }

}  // extern "C"
