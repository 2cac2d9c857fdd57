/* The prefill kernels for 64- and 256-dim heads, behind
 * tq_launch_prefill_other (see tq_prefill.hip). */
#define TQ_PREFILL_OTHER
#include "tq_prefill.hip"
