// A host program that drives libpa through include/pa.h alone: the HIP
// runtime for device memory and a stream, no Python. It reads one decode
// step's inputs from a directory of raw files, runs pa_write_kv and then
// pa_decode_balanced on one stream with a caller-owned workspace (its
// contents need not be initialised), then the same attention as split-K
// partials plus their merge in a workspace sized by pa_splitk_workspace_bytes,
// and writes both outputs and both caches back to the directory.
// It also checks one error path: a head count that is not a multiple of the
// KV head count must be refused with PA_ERR_SHAPE before anything launches.
// tests/test_gpu_c_abi.py builds the inputs and compares the results with the
// oracle.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "pa.h"

#define CHECK_HIP(x)                                                                  \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      std::exit(2);                                                                   \
    }                                                                                 \
  } while (0)
#define CHECK_PA(x)                                                                       \
  do {                                                                                    \
    pa_status s_ = (x);                                                                   \
    if (s_ != PA_OK) {                                                                    \
      std::fprintf(stderr, "%s:%d: %s (%d)\n", __FILE__, __LINE__, pa_status_str(s_), s_); \
      std::exit(3);                                                                       \
    }                                                                                     \
  } while (0)

static std::vector<char> read_file(const std::string& path) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) {
    std::fprintf(stderr, "cannot open %s\n", path.c_str());
    std::exit(4);
  }
  std::fseek(f, 0, SEEK_END);
  const long n = std::ftell(f);
  std::fseek(f, 0, SEEK_SET);
  std::vector<char> buf(n > 0 ? (size_t)n : 0);
  if (n > 0 && std::fread(buf.data(), 1, (size_t)n, f) != (size_t)n) std::exit(4);
  std::fclose(f);
  return buf;
}

static void write_file(const std::string& path, const void* data, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f || std::fwrite(data, 1, bytes, f) != bytes) std::exit(5);
  std::fclose(f);
}

static void* to_device(const std::vector<char>& h) {
  void* d = nullptr;
  CHECK_HIP(hipMalloc(&d, h.size() ? h.size() : 1));
  if (!h.empty()) CHECK_HIP(hipMemcpy(d, h.data(), h.size(), hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 1;
  }
  const std::string dir = argv[1];
  int num_blocks, block_size, hkv, d, dtype, num_seqs, num_heads, max_blocks, max_seq_len;
  float scale;
  {
    FILE* f = std::fopen((dir + "/meta.txt").c_str(), "r");
    if (!f || std::fscanf(f, "%d %d %d %d %d %d %d %d %d %f", &num_blocks, &block_size, &hkv, &d,
                          &dtype, &num_seqs, &num_heads, &max_blocks, &max_seq_len, &scale) != 10)
      return 4;
    std::fclose(f);
  }
  const auto k_cache = read_file(dir + "/k_cache.bin"), v_cache = read_file(dir + "/v_cache.bin");
  void* dk = to_device(k_cache);
  void* dv = to_device(v_cache);
  void* dkn = to_device(read_file(dir + "/k_new.bin"));
  void* dvn = to_device(read_file(dir + "/v_new.bin"));
  void* dslot = to_device(read_file(dir + "/slot_mapping.bin"));
  const auto q = read_file(dir + "/q.bin");
  void* dq = to_device(q);
  void* dbt = to_device(read_file(dir + "/block_table.bin"));
  void* dlens = to_device(read_file(dir + "/seq_lens.bin"));
  void* dout = nullptr;
  CHECK_HIP(hipMalloc(&dout, q.size()));

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  pa_kv_cache cache = {dk, dv, num_blocks, block_size, hkv, d, (pa_dtype)dtype, 1.0f, 1.0f};

  // the error path: nothing is launched for an invalid head count
  if (pa_decode(&cache, dout, dq, (const int32_t*)dbt, (const int32_t*)dlens, num_seqs,
                num_heads + 1, max_blocks, max_seq_len, scale, stream) != PA_ERR_SHAPE) {
    std::fprintf(stderr, "an invalid head count was not refused\n");
    return 6;
  }

  CHECK_PA(pa_write_kv(&cache, dkn, dvn, (const int64_t*)dslot, num_seqs, stream));
  const size_t ws_bytes = pa_decode_balanced_workspace_bytes(&cache, num_seqs, num_heads);
  if (ws_bytes == 0) return 7;
  void* ws = nullptr;
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_PA(pa_decode_balanced(&cache, dout, dq, (const int32_t*)dbt, (const int32_t*)dlens,
                              num_seqs, num_heads, max_blocks, max_seq_len, scale, ws, ws_bytes,
                              stream));
  // the same step's attention again as split-K partials and their LSE merge
  // [P1 §07], both partial arrays carved from one workspace of
  // pa_splitk_workspace_bytes bytes (lse_part at float offset B*Hq*S*D)
  const int split_tokens = 64;
  const int splits = pa_splitk_num_splits(max_seq_len, split_tokens);
  const size_t sk_bytes =
      pa_splitk_workspace_bytes(num_seqs, num_heads, d, max_seq_len, split_tokens);
  const size_t o_floats = (size_t)num_seqs * num_heads * splits * d;
  if (splits <= 0 || sk_bytes != (o_floats + (size_t)num_seqs * num_heads * splits) * 4)
    return 8;
  void* sk = nullptr;
  CHECK_HIP(hipMalloc(&sk, sk_bytes));
  float* o_part = static_cast<float*>(sk);
  float* lse_part = o_part + o_floats;
  void* dout_sk = nullptr;
  CHECK_HIP(hipMalloc(&dout_sk, q.size()));
  CHECK_PA(pa_decode_splitk(&cache, o_part, lse_part, dq, (const int32_t*)dbt,
                            (const int32_t*)dlens, num_seqs, num_heads, max_blocks, max_seq_len,
                            split_tokens, scale, stream));
  CHECK_PA(pa_lse_merge(dout_sk, nullptr, o_part, lse_part, (const int32_t*)dlens, num_seqs,
                        num_heads, d, max_seq_len, split_tokens, (pa_dtype)dtype, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  std::vector<char> out(q.size()), out_sk(q.size()), k_after(k_cache.size()),
      v_after(v_cache.size());
  CHECK_HIP(hipMemcpy(out.data(), dout, out.size(), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out_sk.data(), dout_sk, out_sk.size(), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(k_after.data(), dk, k_after.size(), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(v_after.data(), dv, v_after.size(), hipMemcpyDeviceToHost));
  write_file(dir + "/out.bin", out.data(), out.size());
  write_file(dir + "/out_splitk.bin", out_sk.data(), out_sk.size());
  write_file(dir + "/k_after.bin", k_after.data(), k_after.size());
  write_file(dir + "/v_after.bin", v_after.data(), v_after.size());

  for (void* p : {dk, dv, dkn, dvn, dslot, dq, dbt, dlens, dout, ws, sk, dout_sk}) CHECK_HIP(hipFree(p));
  CHECK_HIP(hipStreamDestroy(stream));
  std::printf("ok %d requests\n", num_seqs);
  return 0;
}
