"""CPU oracle of the ThriftAttention forward pass (test infrastructure only)."""
