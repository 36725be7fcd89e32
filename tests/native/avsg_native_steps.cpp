// A native caller of libavsg: plain C ABI, HIP runtime memory, no Python or
// torch.  Runs a few decode steps of a small workload (bucketed LRU) whose
// inputs follow simple closed formulas (so that a test can rebuild them
// exactly) and writes the slot table, stamps, hit counts and outputs of every
// step to a file.  The first steps run directly; one step is then captured
// in a HIP graph and the graph is replayed for the remaining steps, with the
// next step's inputs copied into the same device buffers before each replay
// (the step counter lives in the workspace, so the replays count on).
//
//   avsg_native_steps <out_file>
//
// Inputs, for unit u, entry e, element i, step t, query head h:
//   host_kv[u][e][i] = bf16 of ((u * 7 + e * 3 + i) % 17 - 8) / 8
//   q[b][0][h][i]    = bf16 of ((b * 5 + h * 11 + i + t) % 13 - 6) / 8
//   sel[u][0][j]     = (j * 3 + t * 5 + u) % N, sorted ascending (k distinct
//                      ids: 3 is coprime with N)
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/avsg.h"

static uint16_t bf16_of(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);  // exact: every value used here is a multiple of 1/8 in [-1, 1]
}

#define CHECK(x)                                                             \
  do {                                                                       \
    if (!(x)) {                                                              \
      fprintf(stderr, "failed: %s (line %d)\n", #x, __LINE__);               \
      return 1;                                                              \
    }                                                                        \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s <out_file>\n", argv[0]);
    return 2;
  }
  const int B = 2, Hkv = 2, G = 4, N = 1000, k = 100, S = 300, steps = 6, D = 128;
  avsg_config cfg;
  memset(&cfg, 0, sizeof(cfg));
  cfg.batch = B;
  cfg.n_kv_heads = Hkv;
  cfg.n_q_heads = Hkv * G;
  cfg.n_q_tokens = 1;
  cfg.head_dim_qk = D;
  cfg.head_dim_v = D;
  cfg.kv_layout = AVSG_KV_SPLIT;
  cfg.n_entries = N;
  cfg.tokens_per_entry = 1;
  cfg.k = k;
  cfg.n_slots = S;
  cfg.policy = AVSG_POLICY_BUCKET_LRU;
  cfg.lifetime_L = 3;
  cfg.n_buckets = 8;
  cfg.softmax_scale = 1.0f / 11.313708498984761f;
  cfg.attn_split_rows = 0;  // the library's choice
  cfg.bucket_width = 1;
  CHECK(avsg_check_config(&cfg) == AVSG_OK);
  const int units = B * Hkv, row = 2 * D, Hq = Hkv * G;

  size_t ws_bytes = avsg_workspace_bytes(&cfg);
  CHECK(ws_bytes > 0);
  void *ws, *buf, *slots, *life, *sel_d, *q_d, *out_d, *hit, *ss, *nh, *nm, *ne, *us;
  CHECK(hipMalloc(&ws, ws_bytes) == hipSuccess);
  CHECK(hipMalloc(&buf, (size_t)units * S * row * 2) == hipSuccess);
  CHECK(hipMalloc(&slots, (size_t)units * S * 4) == hipSuccess);
  CHECK(hipMalloc(&life, (size_t)units * S * 4) == hipSuccess);
  CHECK(hipMalloc(&sel_d, (size_t)units * k * 4) == hipSuccess);
  CHECK(hipMalloc(&q_d, (size_t)B * Hq * D * 2) == hipSuccess);
  CHECK(hipMalloc(&out_d, (size_t)B * Hq * D * 4) == hipSuccess);
  CHECK(hipMalloc(&hit, (size_t)units * k) == hipSuccess);
  CHECK(hipMalloc(&ss, (size_t)units * k * 4) == hipSuccess);
  CHECK(hipMalloc(&nh, units * 4) == hipSuccess);
  CHECK(hipMalloc(&nm, units * 4) == hipSuccess);
  CHECK(hipMalloc(&ne, units * 4) == hipSuccess);
  CHECK(hipMalloc(&us, units * 4) == hipSuccess);
  void* host = nullptr;
  CHECK(avsg_host_alloc((size_t)units * N * row * 2, 0, &host) == AVSG_OK);
  uint16_t* hk = (uint16_t*)host;
  for (int u = 0; u < units; ++u)
    for (int e = 0; e < N; ++e)
      for (int i = 0; i < row; ++i)
        hk[((size_t)u * N + e) * row + i] = bf16_of(((u * 7 + e * 3 + i) % 17 - 8) / 8.0f);

  hipStream_t stream = nullptr;
  CHECK(hipStreamCreate(&stream) == hipSuccess);
  avsg_ctx* ctx = nullptr;
  CHECK(avsg_create(&cfg, stream, ws, ws_bytes, &ctx) == AVSG_OK);
  CHECK(avsg_reset(ctx, (int32_t*)slots, (int32_t*)life) == AVSG_OK);
  avsg_hit_stats hs = {(uint8_t*)hit, (int32_t*)ss, (int32_t*)nh, (int32_t*)nm, (int32_t*)ne,
                       (int32_t*)us};
  FILE* f = fopen(argv[1], "wb");
  CHECK(f != nullptr);
  std::vector<int32_t> sel(units * k), st(units * S), lf(units * S), cnt(units);
  std::vector<uint16_t> q((size_t)B * Hq * D);
  std::vector<float> out((size_t)B * Hq * D);
  const int eager_steps = 3;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  for (int t = 0; t < steps; ++t) {
    for (int u = 0; u < units; ++u) {
      for (int j = 0; j < k; ++j) sel[u * k + j] = (j * 3 + t * 5 + u) % N;
      std::sort(sel.begin() + u * k, sel.begin() + (u + 1) * k);
    }
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hq; ++h)
        for (int i = 0; i < D; ++i)
          q[((size_t)b * Hq + h) * D + i] = bf16_of(((b * 5 + h * 11 + i + t) % 13 - 6) / 8.0f);
    CHECK(hipMemcpyAsync(sel_d, sel.data(), sel.size() * 4, hipMemcpyHostToDevice, stream) ==
          hipSuccess);
    CHECK(hipMemcpyAsync(q_d, q.data(), q.size() * 2, hipMemcpyHostToDevice, stream) ==
          hipSuccess);
    CHECK(hipStreamSynchronize(stream) == hipSuccess);
    if (t < eager_steps) {
      CHECK(avsg_step(ctx, (int32_t*)sel_d, (uint16_t*)q_d, hk, (uint16_t*)buf, (int32_t*)slots,
                      (int32_t*)life, (float*)out_d, &hs) == AVSG_OK);
    } else {
      if (!exec) {  // recorded once, not run while recording
        CHECK(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal) == hipSuccess);
        CHECK(avsg_step(ctx, (int32_t*)sel_d, (uint16_t*)q_d, hk, (uint16_t*)buf,
                        (int32_t*)slots, (int32_t*)life, (float*)out_d, &hs) == AVSG_OK);
        CHECK(hipStreamEndCapture(stream, &graph) == hipSuccess);
        CHECK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess);
        CHECK(avsg_get_step(ctx) == eager_steps);
      }
      CHECK(hipGraphLaunch(exec, stream) == hipSuccess);
    }
    CHECK(hipStreamSynchronize(stream) == hipSuccess);
    CHECK(avsg_get_step(ctx) == t + 1);
    CHECK(hipMemcpy(st.data(), slots, st.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(hipMemcpy(lf.data(), life, lf.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(hipMemcpy(cnt.data(), nh, cnt.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(hipMemcpy(out.data(), out_d, out.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
    fwrite(st.data(), 4, st.size(), f);
    fwrite(lf.data(), 4, lf.size(), f);
    fwrite(cnt.data(), 4, cnt.size(), f);
    fwrite(out.data(), 4, out.size(), f);
  }
  fclose(f);
  CHECK(avsg_last_error(ctx) == AVSG_OK);
  CHECK(hipGraphExecDestroy(exec) == hipSuccess);
  CHECK(hipGraphDestroy(graph) == hipSuccess);
  CHECK(avsg_destroy(ctx) == AVSG_OK);
  CHECK(hipStreamDestroy(stream) == hipSuccess);
  CHECK(avsg_host_free(host) == AVSG_OK);
  for (void* p : {ws, buf, slots, life, sel_d, q_d, out_d, hit, ss, nh, nm, ne, us})
    CHECK(hipFree(p) == hipSuccess);
  printf("native caller: %d steps, %d of them replayed from a graph\n", steps,
         steps - eager_steps);
  return 0;
}
