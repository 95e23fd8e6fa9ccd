/* An end-to-end use of libpa from C, with no Python and no PyTorch: HIP device
 * memory, the host block manager (pa_blocks.h), prompts written with
 * pa_cache_append, a fork that shares a sequence's blocks, one decode step through
 * the executor (pa_step.h, which carries out the copy-on-write, the append and the
 * decode), the same decode once more through pa_decode (pa.h) with the
 * executor's device tables, and once more through pa_decode_append with the step's
 * new rows (which rewrites them into the slots they already hold).  Everything the
 * device computed, and every input, is written to the file named on the command line
 * for a test to check against the oracle.
 *
 * Build: gcc -std=c11 -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include -Iinclude
 *        c_abi_demo.c -Lpaged_kv_cache_414_amd -lpa -L/opt/rocm/lib -lamdhip64
 * Usage: c_abi_demo OUT_FILE
 *
 * OUT_FILE: int32 header [H, D, BS, NB, S, MB, prompt tokens T, copies C], then, in
 * order: int32 prompt slots [T]; float prompt K, V [T, H, D]; float q, new K, new V
 * [S, H, D]; int32 step slots [S]; int32 copy pairs [C, 2]; int32 block tables
 * [S, MB]; int32 context lengths [S]; float out (executor) [S, H, D]; float out
 * (pa_decode) [S, H, D]; float out (pa_decode_append) [S, H, D]; float K pool, V pool
 * [NB, H, BS, D] after all three.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pa.h"
#include "pa_blocks.h"
#include "pa_step.h"

enum { H = 4, D = 64, BS = 16, NB = 32, S = 4, MB = 8 };

static void die(const char* what, const char* why) {
  fprintf(stderr, "c_abi_demo: %s: %s\n", what, why);
  exit(1);
}
#define HIP_OK(x)                                   \
  do {                                              \
    hipError_t err_ = (x);                          \
    if (err_ != hipSuccess) die(#x, hipGetErrorString(err_)); \
  } while (0)
#define PA_OK_(x)                                   \
  do {                                              \
    pa_status st_ = (x);                            \
    if (st_ != PA_OK) die(#x, pa_last_error());     \
  } while (0)

/* xorshift64* (Vigna, "An experimental exploration of Marsaglia's xorshift
 * generators, scrambled", 2016), mapped to [-1, 1) */
static uint64_t rng_state = 0x2545F4914F6CDD1Dull;
static float next_value(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  const uint64_t x = rng_state * 0x2545F4914F6CDD1Dull;
  return (float)((double)(x >> 40) / 16777216.0 * 2.0 - 1.0);
}

static float* fill(size_t n) {
  float* p = (float*)malloc(n * sizeof(float));
  if (!p) die("malloc", "out of memory");
  for (size_t i = 0; i < n; ++i) p[i] = next_value();
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes));
  HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void put(FILE* f, const void* p, size_t bytes) {
  if (bytes && fwrite(p, 1, bytes, f) != bytes) die("fwrite", "short write");
}

int main(int argc, char** argv) {
  if (argc != 2) die("usage", "c_abi_demo OUT_FILE");
  const size_t row = (size_t)H * D;
  const size_t pool_elems = (size_t)NB * H * BS * D;

  /* three prompts of 20, 33 and 16 tokens, admitted together */
  pa_block_manager* bm = pa_bm_create(NB, BS, 11);
  if (!bm) die("pa_bm_create", pa_last_error());
  const int64_t ids[3] = {0, 1, 2};
  const int32_t lens[3] = {20, 33, 16};
  const int32_t T = lens[0] + lens[1] + lens[2];
  int32_t* slots = (int32_t*)malloc(T * sizeof(int32_t));
  PA_OK_(pa_bm_add_sequences(bm, ids, lens, 3, slots));
  float* pk = fill(T * row);
  float* pv = fill(T * row);

  float *kc = NULL, *vc = NULL;
  HIP_OK(hipMalloc((void**)&kc, pool_elems * sizeof(float)));
  HIP_OK(hipMalloc((void**)&vc, pool_elems * sizeof(float)));
  HIP_OK(hipMemset(kc, 0, pool_elems * sizeof(float)));
  HIP_OK(hipMemset(vc, 0, pool_elems * sizeof(float)));
  void* d_pk = to_device(pk, T * row * sizeof(float));
  void* d_pv = to_device(pv, T * row * sizeof(float));
  void* d_slots = to_device(slots, T * sizeof(int32_t));
  PA_OK_(pa_cache_append(kc, vc, d_pk, d_pv, (const int32_t*)d_slots, T, H, D, BS, NB, PA_F32, NULL));

  /* sequence 3 shares every block of sequence 0: its partly filled last block is
   * copied when the first of the two writes into it */
  PA_OK_(pa_bm_fork(bm, 0, 3));

  /* one decode step of the four sequences through the executor */
  const pa_step_config cfg = {H, D, PA_F32, S, MB, 0, 0};
  pa_step_engine* eng = pa_step_create(bm, &cfg, kc, vc);
  if (!eng) die("pa_step_create", pa_last_error());
  float* q = fill(S * row);
  float* nk = fill(S * row);
  float* nv = fill(S * row);
  void* d_q = to_device(q, S * row * sizeof(float));
  void* d_nk = to_device(nk, S * row * sizeof(float));
  void* d_nv = to_device(nv, S * row * sizeof(float));
  void *d_out = NULL, *d_out2 = NULL, *d_out3 = NULL;
  HIP_OK(hipMalloc(&d_out, S * row * sizeof(float)));
  HIP_OK(hipMalloc(&d_out2, S * row * sizeof(float)));
  HIP_OK(hipMalloc(&d_out3, S * row * sizeof(float)));
  const int64_t running[S] = {0, 1, 2, 3};
  pa_step_args args;
  memset(&args, 0, sizeof(args));
  args.seq_ids = running;
  args.num_seqs = S;
  args.query = d_q;
  args.new_key = d_nk;
  args.new_value = d_nv;
  args.out = d_out;
  args.scale = 0.125f;
  pa_step_result res;
  PA_OK_(pa_step_run(eng, &args, NULL, &res));
  pa_step_view view;
  PA_OK_(pa_step_last(eng, &view));

  /* the same decode through pa_decode, on the executor's device tables */
  const size_t ws_bytes = pa_decode_workspace_bytes(S, H, D, BS, res.max_context_len, 0);
  void* ws = NULL;
  if (ws_bytes) HIP_OK(hipMalloc(&ws, ws_bytes));
  PA_OK_(pa_decode(d_out2, d_q, kc, vc, view.dev_block_tables, view.dev_context_lens, S, H, D, BS, NB, MB,
                   res.max_context_len, 0.125f, PA_F32, 0, ws, ws_bytes, NULL));
  /* and through pa_decode_append: the new rows go to position context - 1, where the
   * executor already put them */
  PA_OK_(pa_decode_append(d_out3, d_q, kc, vc, d_nk, d_nv, view.dev_block_tables, view.dev_context_lens, S, H,
                          D, BS, NB, MB, res.max_context_len, 0.125f, PA_F32, 0, ws, ws_bytes, NULL));
  HIP_OK(hipDeviceSynchronize());

  float* out = (float*)malloc(S * row * sizeof(float));
  float* out2 = (float*)malloc(S * row * sizeof(float));
  float* out3 = (float*)malloc(S * row * sizeof(float));
  float* kpool = (float*)malloc(pool_elems * sizeof(float));
  float* vpool = (float*)malloc(pool_elems * sizeof(float));
  HIP_OK(hipMemcpy(out, d_out, S * row * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out2, d_out2, S * row * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out3, d_out3, S * row * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(kpool, kc, pool_elems * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(vpool, vc, pool_elems * sizeof(float), hipMemcpyDeviceToHost));

  FILE* f = fopen(argv[1], "wb");
  if (!f) die("fopen", argv[1]);
  const int32_t header[8] = {H, D, BS, NB, S, MB, T, res.num_copies};
  put(f, header, sizeof(header));
  put(f, slots, T * sizeof(int32_t));
  put(f, pk, T * row * sizeof(float));
  put(f, pv, T * row * sizeof(float));
  put(f, q, S * row * sizeof(float));
  put(f, nk, S * row * sizeof(float));
  put(f, nv, S * row * sizeof(float));
  put(f, view.slots, S * sizeof(int32_t));
  put(f, view.copy_pairs, (size_t)res.num_copies * 2 * sizeof(int32_t));
  put(f, view.block_tables, (size_t)S * MB * sizeof(int32_t));
  put(f, view.context_lens, S * sizeof(int32_t));
  put(f, out, S * row * sizeof(float));
  put(f, out2, S * row * sizeof(float));
  put(f, out3, S * row * sizeof(float));
  put(f, kpool, pool_elems * sizeof(float));
  put(f, vpool, pool_elems * sizeof(float));
  fclose(f);

  pa_step_destroy(eng);
  pa_bm_destroy(bm);
  void* bufs[] = {kc, vc, d_pk, d_pv, d_slots, d_q, d_nk, d_nv, d_out, d_out2, d_out3, ws};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) {
    if (bufs[i]) HIP_OK(hipFree(bufs[i]));
  }
  printf("c_abi_demo: %d sequences decoded, %d copy-on-write pair(s)\n", S, res.num_copies);
  return 0;
}
