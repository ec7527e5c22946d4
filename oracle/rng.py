"""Counter-based random draws for the oracle (test infrastructure only).

The HA page draws random columns (section "Algorithm", Algorithm 2) and random
rows of V (section "Method overview") but fixes no generator or seed. To make
two independent implementations draw the same samples, every random number
is a pure function of (seed, purpose, head, node, counter):

    key          = mix64(seed)
    draw(...)    = mix64(key XOR pack(purpose, head, node, counter))
    pack         = purpose << 60 | head << 44 | node << 24 | counter
    mix64(x)     = SplitMix64's output for the state x + 0x9E3779B97F4A7C15

SplitMix64 is the generator of Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014: add the golden-ratio gamma to
the state, then apply two xor-shift-multiply rounds and a final xor-shift.
Field limits: purpose < 16, head < 2**16, node < 2**20, counter < 2**24.
Arithmetic is done on Python integers reduced mod 2**64.
"""

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15

PURPOSE_HYPERPLANE = 1
PURPOSE_UNIFORM = 2
PURPOSE_VNORM = 3


def splitmix64_next(state):
    """One step of SplitMix64: returns (new_state, output)."""
    state = (state + GOLDEN_GAMMA) & MASK64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    z = z ^ (z >> 31)
    return state, z


def mix64(x):
    """The output SplitMix64 gives when its state before the step is x."""
    return splitmix64_next(x & MASK64)[1]


def pack(purpose, head, node, counter):
    if not (0 <= purpose < 16 and 0 <= head < (1 << 16)
            and 0 <= node < (1 << 20) and 0 <= counter < (1 << 24)):
        raise ValueError("counter fields out of range")
    return (purpose << 60) | (head << 44) | (node << 24) | counter


def draw(seed, purpose, head, node, counter):
    """A 64-bit random integer for one (purpose, head, node, counter)."""
    return mix64(mix64(seed) ^ pack(purpose, head, node, counter))
