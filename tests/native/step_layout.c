/* Prints the size and field offsets of the structs of pa_step.h, one per line, so
 * that a test can compare them with the ctypes mirrors of the Python binding. */
#include <stddef.h>
#include <stdio.h>

#include "pa_step.h"

#define F(T, f) printf("%s.%s %zu\n", #T, #f, offsetof(T, f))
#define S(T) printf("%s %zu\n", #T, sizeof(T))

int main(void) {
  S(pa_step_config);
  F(pa_step_config, num_heads); F(pa_step_config, head_dim); F(pa_step_config, dtype);
  F(pa_step_config, max_seqs); F(pa_step_config, max_blocks_per_seq);
  F(pa_step_config, max_admit_tokens); F(pa_step_config, max_groups);
  S(pa_step_args);
  F(pa_step_args, seq_ids); F(pa_step_args, num_seqs); F(pa_step_args, query);
  F(pa_step_args, new_key); F(pa_step_args, new_value); F(pa_step_args, out);
  F(pa_step_args, scale); F(pa_step_args, group_starts); F(pa_step_args, num_groups);
  F(pa_step_args, finished_ids); F(pa_step_args, num_finished); F(pa_step_args, admit_ids);
  F(pa_step_args, admit_lens); F(pa_step_args, num_admit); F(pa_step_args, prompt_key);
  F(pa_step_args, prompt_value);
  S(pa_step_result);
  F(pa_step_result, num_copies); F(pa_step_result, num_admitted);
  F(pa_step_result, admitted_tokens); F(pa_step_result, max_context_len);
  F(pa_step_result, max_prefix_len); F(pa_step_result, max_suffix_len);
  F(pa_step_result, max_group_size);
  S(pa_step_view);
  F(pa_step_view, num_seqs); F(pa_step_view, num_groups); F(pa_step_view, result);
  F(pa_step_view, slots); F(pa_step_view, positions); F(pa_step_view, copy_pairs);
  F(pa_step_view, block_tables); F(pa_step_view, context_lens); F(pa_step_view, group_starts);
  F(pa_step_view, prefix_lens); F(pa_step_view, admit_slots); F(pa_step_view, dev_block_tables);
  F(pa_step_view, dev_context_lens); F(pa_step_view, dev_group_starts);
  F(pa_step_view, dev_prefix_lens); F(pa_step_view, workspace); F(pa_step_view, workspace_bytes);
  F(pa_step_view, hints);
  return 0;
}
