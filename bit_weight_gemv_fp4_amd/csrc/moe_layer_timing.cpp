// moe_layer_timing.cpp -- a stand-alone timing program for one MoE decode layer
// through the library's C ABI only (moe_route_gemv), small enough to run under
// rocprofv3's counter collection: its set-up issues no kernel launches besides
// fills, so a --pmc run profiles little but the layer's own kernels.
//
// Shapes: the Ling-3.0 article's MoE layer (sec. 3): 512 routed experts + one
// shared, top-8, hidden 2560, expert width 768, MXFP4 weights.  The packed
// matrices are filled with one byte pattern (any MXFP4 code byte is a valid pair
// of elements; 0x3c as an E8M0 scale is 2^-67, finite), which changes nothing the
// kernels read or skip: the bytes streamed depend only on which experts the
// router picks.  Router logits are seeded uniform values in [-2, 2) from a 32-bit
// linear congruential generator, a fresh row per token and layer.
//
//   moe_layer_timing [M] [layers] [reps]      (defaults 1 16 20)
//
// Prints the mean time per layer over `reps` passes of `layers` distinct layers
// (each layer's weights are read once per pass, so nothing stays in the caches),
// the mean realised union of experts per layer (the device's picks, checked
// against a host top-k of the same logits), and the weight bytes that union
// implies: (union + shared) x (2 x gate/up + down packed bytes).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <set>
#include <vector>

#include "../../include/fp4gemv.h"

#define CK(x)                                                                                      \
  do {                                                                                             \
    hipError_t e_ = (x);                                                                           \
    if (e_ != hipSuccess) {                                                                        \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);          \
      std::exit(1);                                                                                \
    }                                                                                              \
  } while (0)
#define CF(x)                                                                                      \
  do {                                                                                             \
    int32_t r_ = (x);                                                                              \
    if (r_ != 0) {                                                                                 \
      std::fprintf(stderr, "library error %s at line %d\n", fp4g_status_string(r_), __LINE__);     \
      std::exit(1);                                                                                \
    }                                                                                              \
  } while (0)

namespace {
constexpr int kExperts = 512, kTopK = 8, kHidden = 2560, kFF = 768;

fp4g_weight view(const uint8_t* p, uint64_t bytes, int d_out, int d_in) {
  fp4g_weight w{};
  w.format = FP4G_MXFP4;
  w.layout_tag = FP4G_LAYOUT_TILE64x256;
  w.d_out = d_out;
  w.d_in = d_in;
  w.packed = p;
  w.packed_bytes = bytes;
  w.tensor_scale = 1.0f;
  return w;
}

// The top_k expert ids of one logit row: descending value, ties to the lower index.
std::vector<int> host_topk(const float* row) {
  std::vector<int> idx(kExperts);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return row[a] > row[b]; });
  idx.resize(kTopK);
  return idx;
}
}  // namespace

int main(int argc, char** argv) {
  const int M = argc > 1 ? std::atoi(argv[1]) : 1;
  const int NL = argc > 2 ? std::atoi(argv[2]) : 16;
  const int reps = argc > 3 ? std::atoi(argv[3]) : 20;
  if (M < 1 || M > FP4G_MAX_M_WIDE || NL < 1 || NL > 64 || reps < 1) {
    std::fprintf(stderr, "usage: moe_layer_timing [M 1..16] [layers 1..64] [reps >= 1]\n");
    return 2;
  }
  const uint64_t pg = fp4g_packed_bytes(FP4G_MXFP4, kFF, kHidden);
  const uint64_t pd = fp4g_packed_bytes(FP4G_MXFP4, kHidden, kFF);
  std::printf("MoE layer: %d experts + shared, top-%d, MXFP4 gate/up %dx%d, down %dx%d; M=%d, %d layers, %d passes\n",
              kExperts, kTopK, kFF, kHidden, kHidden, kFF, M, NL, reps);

  std::vector<fp4g_moe> layers(NL);
  std::vector<uint8_t*> bufs;
  for (int l = 0; l < NL; ++l) {
    uint8_t* b[3];
    const uint64_t st[3] = {pg, pg, pd};
    for (int k = 0; k < 3; ++k) {  // expert kExperts of each buffer is the shared expert
      CK(hipMalloc(&b[k], (kExperts + 1) * st[k]));
      CK(hipMemset(b[k], 0x3c, (kExperts + 1) * st[k]));
      bufs.push_back(b[k]);
    }
    fp4g_moe& mo = layers[l];
    mo = fp4g_moe{};
    mo.num_experts = kExperts;
    mo.top_k = kTopK;
    mo.hidden = kHidden;
    mo.d_ff = kFF;
    mo.gate = view(b[0], kExperts * pg, kFF, kHidden);
    mo.up = view(b[1], kExperts * pg, kFF, kHidden);
    mo.down = view(b[2], kExperts * pd, kHidden, kFF);
    mo.stride_gate = pg;
    mo.stride_up = pg;
    mo.stride_down = pd;
    mo.has_shared = 1;
    mo.act = FP4G_ACT_BF16;
    mo.sh_gate = view(b[0] + kExperts * pg, pg, kFF, kHidden);
    mo.sh_up = view(b[1] + kExperts * pg, pg, kFF, kHidden);
    mo.sh_down = view(b[2] + kExperts * pd, pd, kHidden, kFF);
  }

  std::vector<float> lg((size_t)NL * M * kExperts);
  uint32_t s = 12345u;
  for (float& v : lg) {
    s = s * 1664525u + 1013904223u;
    v = (float)((s >> 8) & 0xffffu) / 65536.0f * 4.0f - 2.0f;
  }
  uint16_t* X;
  float *logits, *Y, *tw;
  int* ids;
  CK(hipMalloc(&X, (size_t)M * kHidden * 2));
  CK(hipMemset(X, 0x3c, (size_t)M * kHidden * 2));  // bf16 1.1719 everywhere
  CK(hipMalloc(&logits, lg.size() * 4));
  CK(hipMemcpy(logits, lg.data(), lg.size() * 4, hipMemcpyHostToDevice));
  CK(hipMalloc(&Y, (size_t)M * kHidden * 4));
  CK(hipMalloc(&ids, (size_t)NL * M * kTopK * 4));
  CK(hipMalloc(&tw, (size_t)M * kTopK * 4));
  const uint64_t wsb = fp4g_workspace_bytes(FP4G_OP_MOE, &layers[0], M);
  uint8_t* ws;
  CK(hipMalloc(&ws, wsb));
  CK(hipMemset(ws, 0, wsb));
  hipStream_t st;
  CK(hipStreamCreate(&st));

  auto pass = [&]() {
    for (int l = 0; l < NL; ++l)
      CF(moe_route_gemv(&layers[l], X, logits + (size_t)l * M * kExperts, M, Y, ids + (size_t)l * M * kTopK, tw,
                        nullptr, ws, wsb, st));
  };
  for (int r = 0; r < 3; ++r) pass();
  CK(hipStreamSynchronize(st));

  // the device's picks against a host top-k of the same logits, and the union they make
  std::vector<int> dev_ids((size_t)NL * M * kTopK);
  CK(hipMemcpy(dev_ids.data(), ids, dev_ids.size() * 4, hipMemcpyDeviceToHost));
  double slots = 0;
  for (int l = 0; l < NL; ++l) {
    std::set<int> uni;
    for (int m = 0; m < M; ++m) {
      const std::vector<int> want = host_topk(lg.data() + ((size_t)l * M + m) * kExperts);
      for (int j = 0; j < kTopK; ++j) {
        const int got = dev_ids[((size_t)l * M + m) * kTopK + j];
        if (got != want[j]) {
          std::fprintf(stderr, "layer %d token %d pick %d: device %d, host %d\n", l, m, j, got, want[j]);
          return 1;
        }
        uni.insert(got);
      }
    }
    slots += (double)uni.size() + 1;  // + the shared expert
  }
  slots /= NL;

  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  CK(hipEventRecord(e0, st));
  for (int r = 0; r < reps; ++r) pass();
  CK(hipEventRecord(e1, st));
  CK(hipEventSynchronize(e1));
  float ms = 0;
  CK(hipEventElapsedTime(&ms, e0, e1));
  const double us = ms * 1e3 / ((double)reps * NL);
  const double bytes = slots * (2.0 * pg + pd);
  std::printf("picks match the host top-%d on every layer and token\n", kTopK);
  std::printf("realised experts per layer (union + shared): %.2f -> weight bytes %.3f MB per layer\n", slots,
              bytes / 1e6);
  std::printf("%.2f us per layer -> %.1f GB/s of weight bytes\n", us, bytes / (us * 1e3));

  CK(hipStreamDestroy(st));
  for (uint8_t* b : bufs) CK(hipFree(b));
  CK(hipFree(X));
  CK(hipFree(logits));
  CK(hipFree(Y));
  CK(hipFree(ids));
  CK(hipFree(tw));
  CK(hipFree(ws));
  return 0;
}
