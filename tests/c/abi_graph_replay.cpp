// abi_graph_replay.cpp -- a C++/HIP caller of libnvfp4g.so with no PyTorch
// (test infrastructure).  Every buffer comes from hipMalloc; one call of
// nvfp4_group_quantize_graphsafe is captured into a hipGraph on the
// program's own stream, and the graph is replayed once per routing in the
// input file.  Before each replay the device offsets are rewritten, the
// status word is cleared and every output is filled with a sentinel byte
// (all outside the graph); after it the outputs and the status are copied
// back.  The library's host-side checks are exercised first: a call with
// K = 15 must be refused with NVFP4G_EINVAL before anything is launched; and
// the captured graph must hold kernel nodes only (no memset nodes).
//
//   usage: abi_graph_replay <in.bin> <out.bin>
//   in.bin  (little-endian): int64 m_cap, k, E, R; int32 offs[R][E]
//           (inclusive row ends); uint16 x[m_cap][k] (bf16 bits)
//   out.bin: per replay: int32 status; float row_amax[m_cap];
//           float col_amax[E*k]; uint8 row_data[m_cap*k/2];
//           uint8 row_scale[m_cap*k/16]; uint8 col_data[m_cap*k/2];
//           uint8 col_scale[m_cap*k/16]
// Exit status 0 on success, 1 on any error (printed).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "nvfp4_group.h"

#define HIP_OK(call)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) {                                                               \
      std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));              \
      return 1;                                                                           \
    }                                                                                     \
  } while (0)

constexpr unsigned char kSentinel = 0xA5;

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s <in.bin> <out.bin>\n", argv[0]);
    return 1;
  }
  std::FILE* in = std::fopen(argv[1], "rb");
  if (!in) {
    std::fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int64_t hdr[4];
  if (std::fread(hdr, sizeof(int64_t), 4, in) != 4) return 1;
  const int64_t m_cap = hdr[0], k = hdr[1], E = hdr[2], R = hdr[3];
  if (m_cap <= 0 || k <= 0 || E <= 0 || R <= 0 || m_cap % 128 || k % 16 || E > 4096 || R > 1024) {
    std::fprintf(stderr, "bad header\n");
    return 1;
  }
  std::vector<int32_t> offs((size_t)(R * E));
  std::vector<uint16_t> x((size_t)(m_cap * k));
  if (std::fread(offs.data(), sizeof(int32_t), offs.size(), in) != offs.size() ||
      std::fread(x.data(), sizeof(uint16_t), x.size(), in) != x.size()) {
    std::fprintf(stderr, "short input\n");
    return 1;
  }
  std::fclose(in);

  const size_t n_row_amax = (size_t)m_cap, n_col_amax = (size_t)(E * k);
  const size_t n_data = (size_t)(m_cap * k / 2), n_scale = (size_t)(m_cap * k / 16);
  uint16_t* d_x;
  float *d_row_amax, *d_col_amax;
  uint8_t *d_row_data, *d_row_scale, *d_col_data, *d_col_scale;
  int32_t *d_offs, *d_status;
  HIP_OK(hipMalloc(&d_x, x.size() * sizeof(uint16_t)));
  HIP_OK(hipMalloc(&d_row_amax, n_row_amax * sizeof(float)));
  HIP_OK(hipMalloc(&d_col_amax, n_col_amax * sizeof(float)));
  HIP_OK(hipMalloc(&d_row_data, n_data));
  HIP_OK(hipMalloc(&d_row_scale, n_scale));
  HIP_OK(hipMalloc(&d_col_data, n_data));
  HIP_OK(hipMalloc(&d_col_scale, n_scale));
  HIP_OK(hipMalloc(&d_offs, (size_t)E * sizeof(int32_t)));
  HIP_OK(hipMalloc(&d_status, sizeof(int32_t)));
  HIP_OK(hipMemcpy(d_x, x.data(), x.size() * sizeof(uint16_t), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_offs, offs.data(), (size_t)E * sizeof(int32_t), hipMemcpyHostToDevice));
  HIP_OK(hipMemset(d_status, 0, sizeof(int32_t)));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  // host-side refusal: K not a multiple of 16, nothing launched
  const int bad = nvfp4_group_quantize_graphsafe(d_x, m_cap, 15, (int32_t)E, d_offs, d_row_amax, d_col_amax,
                                                 d_row_data, d_row_scale, d_col_data, d_col_scale, d_status,
                                                 stream);
  if (bad != NVFP4G_EINVAL) {
    std::fprintf(stderr, "K = 15 gave %d (%s), expected NVFP4G_EINVAL\n", bad, nvfp4_group_strerror(bad));
    return 1;
  }
  std::printf("refused K = 15: %s\n", nvfp4_group_strerror(bad));

  // one capture of the whole path
  hipGraph_t graph;
  hipGraphExec_t exec;
  HIP_OK(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
  const int rc = nvfp4_group_quantize_graphsafe(d_x, m_cap, k, (int32_t)E, d_offs, d_row_amax, d_col_amax,
                                                d_row_data, d_row_scale, d_col_data, d_col_scale, d_status,
                                                stream);
  HIP_OK(hipStreamEndCapture(stream, &graph));
  if (rc != NVFP4G_OK) {
    std::fprintf(stderr, "capture: %s\n", nvfp4_group_strerror(rc));
    return 1;
  }
  HIP_OK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
  // every node must be a kernel: the amax zero-fill is a kernel, never a
  // memset node
  size_t nodes = 0;
  HIP_OK(hipGraphGetNodes(graph, nullptr, &nodes));
  std::vector<hipGraphNode_t> list(nodes);
  HIP_OK(hipGraphGetNodes(graph, list.data(), &nodes));
  size_t kernels = 0;
  for (size_t i = 0; i < nodes; ++i) {
    hipGraphNodeType type;
    HIP_OK(hipGraphNodeGetType(list[i], &type));
    kernels += type == hipGraphNodeTypeKernel;
  }
  std::printf("captured %zu graph nodes, %zu kernels\n", nodes, kernels);
  if (nodes == 0 || kernels != nodes) {
    std::fprintf(stderr, "the capture holds nodes other than kernels\n");
    return 1;
  }

  std::FILE* out = std::fopen(argv[2], "wb");
  if (!out) {
    std::fprintf(stderr, "cannot open %s\n", argv[2]);
    return 1;
  }
  std::vector<float> h_row_amax(n_row_amax), h_col_amax(n_col_amax);
  std::vector<uint8_t> h_data(n_data), h_scale(n_scale);
  for (int64_t r = 0; r < R; ++r) {
    HIP_OK(hipMemcpy(d_offs, offs.data() + r * E, (size_t)E * sizeof(int32_t), hipMemcpyHostToDevice));
    HIP_OK(hipMemset(d_status, 0, sizeof(int32_t)));
    HIP_OK(hipMemset(d_row_amax, kSentinel, n_row_amax * sizeof(float)));
    HIP_OK(hipMemset(d_col_amax, kSentinel, n_col_amax * sizeof(float)));
    HIP_OK(hipMemset(d_row_data, kSentinel, n_data));
    HIP_OK(hipMemset(d_row_scale, kSentinel, n_scale));
    HIP_OK(hipMemset(d_col_data, kSentinel, n_data));
    HIP_OK(hipMemset(d_col_scale, kSentinel, n_scale));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipGraphLaunch(exec, stream));
    HIP_OK(hipStreamSynchronize(stream));
    int32_t status = -1;
    HIP_OK(hipMemcpy(&status, d_status, sizeof(int32_t), hipMemcpyDeviceToHost));
    std::fwrite(&status, sizeof(int32_t), 1, out);
    HIP_OK(hipMemcpy(h_row_amax.data(), d_row_amax, n_row_amax * sizeof(float), hipMemcpyDeviceToHost));
    std::fwrite(h_row_amax.data(), sizeof(float), n_row_amax, out);
    HIP_OK(hipMemcpy(h_col_amax.data(), d_col_amax, n_col_amax * sizeof(float), hipMemcpyDeviceToHost));
    std::fwrite(h_col_amax.data(), sizeof(float), n_col_amax, out);
    uint8_t* bufs[4] = {d_row_data, d_row_scale, d_col_data, d_col_scale};
    for (int b = 0; b < 4; ++b) {
      std::vector<uint8_t>& h = (b % 2 == 0) ? h_data : h_scale;
      HIP_OK(hipMemcpy(h.data(), bufs[b], h.size(), hipMemcpyDeviceToHost));
      std::fwrite(h.data(), 1, h.size(), out);
    }
    std::printf("replay %lld: status %d\n", (long long)r, status);
  }
  std::fclose(out);
  HIP_OK(hipGraphExecDestroy(exec));
  HIP_OK(hipGraphDestroy(graph));
  HIP_OK(hipStreamDestroy(stream));
  void* bufs[] = {d_x, d_row_amax, d_col_amax, d_row_data, d_row_scale, d_col_data, d_col_scale, d_offs, d_status};
  for (void* p : bufs) HIP_OK(hipFree(p));
  std::printf("done\n");
  return 0;
}
